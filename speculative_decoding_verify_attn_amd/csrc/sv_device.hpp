// sv_device.hpp -- device-side building blocks for gfx950 (wave64).
//
// Wave reductions and scans use DPP lane moves inside 16-lane rows
// (quad_perm, row_shr, row_mirror, row_half_mirror) and the GFX9 row
// broadcasts (row_bcast:15, row_bcast:31) to cross rows; the final value is
// read from lane 63 with v_readlane.  64-bit values move as two 32-bit
// halves.  fp8 E4M3 decode uses the hardware fp8 -> bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// DPP control codes (GFX9 encoding).
enum : int {
    kQuadSwap1 = 0xB1,      // quad_perm [1,0,3,2]
    kQuadSwap2 = 0x4E,      // quad_perm [2,3,0,1]
    kRowShr1 = 0x111,
    kRowShr2 = 0x112,
    kRowShr4 = 0x114,
    kRowShr8 = 0x118,
    kRowMirror = 0x140,
    kRowHalfMirror = 0x141,
    kRowBcast15 = 0x142,
    kRowBcast31 = 0x143,
};

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float identity, float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, identity), __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double identity, double v)
{
    const uint64_t iv = __builtin_bit_cast(uint64_t, identity);
    const uint64_t vv = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)iv, (int)(uint32_t)vv, CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(iv >> 32), (int)(uint32_t)(vv >> 32), CTRL,
                                               ROW_MASK, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ float readlane_f32(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Maximum over the 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_max_f32(float v)
{
    const float id = -__builtin_inff();
    v = fmaxf(v, dpp_f32<kQuadSwap1>(id, v));
    v = fmaxf(v, dpp_f32<kQuadSwap2>(id, v));
    v = fmaxf(v, dpp_f32<kRowHalfMirror>(id, v));
    v = fmaxf(v, dpp_f32<kRowMirror>(id, v));
    v = fmaxf(v, dpp_f32<kRowBcast15, 0xA>(id, v));
    v = fmaxf(v, dpp_f32<kRowBcast31, 0xC>(id, v));
    return readlane_f32(v, 63);
}

// Minimum / maximum of non-negative ints over the wave (in every lane).
__device__ __forceinline__ int wave_min_i32(int v)
{
    const int id = 0x7FFFFFFF;
    v = min(v, __builtin_amdgcn_update_dpp(id, v, kQuadSwap1, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(id, v, kQuadSwap2, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(id, v, kRowHalfMirror, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(id, v, kRowMirror, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(id, v, kRowBcast15, 0xA, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(id, v, kRowBcast31, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_max_i32(int v)
{
    const int id = -0x7FFFFFFF - 1;
    v = max(v, __builtin_amdgcn_update_dpp(id, v, kQuadSwap1, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(id, v, kQuadSwap2, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(id, v, kRowHalfMirror, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(id, v, kRowMirror, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(id, v, kRowBcast15, 0xA, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(id, v, kRowBcast31, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the 64 lanes in double, returned in every lane.  The combination
// order is fixed, so the result is reproducible bit for bit.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<kQuadSwap1>(0.0, v);
    v += dpp_f64<kQuadSwap2>(0.0, v);
    v += dpp_f64<kRowHalfMirror>(0.0, v);
    v += dpp_f64<kRowMirror>(0.0, v);
    v += dpp_f64<kRowBcast15, 0xA>(0.0, v);
    v += dpp_f64<kRowBcast31, 0xC>(0.0, v);
    return readlane_f64(v, 63);
}

// Inclusive prefix sum over lanes 0..63 in double (lane i gets x_0 + .. + x_i).
__device__ __forceinline__ double wave_inclusive_scan_f64(double v)
{
    v += dpp_f64<kRowShr1>(0.0, v);
    v += dpp_f64<kRowShr2>(0.0, v);
    v += dpp_f64<kRowShr4>(0.0, v);
    v += dpp_f64<kRowShr8>(0.0, v);
    v += dpp_f64<kRowBcast15, 0xA>(0.0, v);
    v += dpp_f64<kRowBcast31, 0xC>(0.0, v);
    return v;
}

// Cross-lane exchange with lane ^ mask (ds_bpermute; no LDS storage used).
__device__ __forceinline__ float xor_lane_f32(float v, int mask)
{
    const int lane = __lane_id();
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, v)));
}

// Byte permute: bytes of {hi:lo} selected by `sel` (v_perm_b32).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Low / high bf16 halves of two packed pairs: {a.lo, b.lo} and {a.hi, b.hi}.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// Two floats -> packed bf16 pair (round to nearest even, hardware cvt).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// Four OCP E4M3 codes (bytes 0..3 of `codes`) -> four bf16 values as two
// packed pairs {byte 0, byte 1}, {byte 2, byte 3}.  gfx950's packed
// conversion with a unit scale is exact (every E4M3 value is a bf16 value);
// its scale operand contributes only its exponent, so per-page scales are
// applied separately.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t codes)
{
    uint2 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true));
    return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

}  // namespace sv
