// Shared device helpers for the gfx950 kernels of the decode / verify step:
// storage-type traits (fp32 / fp16 / bf16 values held in memory, fp32
// arithmetic), round-to-nearest-even stores, wave64 shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

constexpr int kWave = 64;

enum DType { F32 = 0, F16 = 1, BF16 = 2, E4M3 = 3, E5M2 = 4 };  // the last two: 8-bit K/V cache only

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the nontemporal (streaming) hint: for data each step reads
// exactly once (weights, K/V pages), so it does not displace reused lines in L2
// and the Infinity Cache. On MI355X this lifts the streaming-read rate by ~7%.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// ---- scalar conversions --------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bfloat16 bits, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}

// fp32 -> binary16 bits; the hardware conversion rounds to nearest even.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    _Float16 h = (_Float16)f;
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

// Storage-type traits. `raw` is the in-memory element; `to_f` widens one
// element; `from_f` rounds an fp32 value to the storage type.
template <int DT> struct St;
template <> struct St<F32> {
    typedef float raw;
    static constexpr int bytes = 4;
    __device__ static __forceinline__ float to_f(raw v) { return v; }
    __device__ static __forceinline__ raw from_f(float f) { return f; }
};
template <> struct St<F16> {
    typedef uint16_t raw;
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float to_f(raw v) { return half_bits_to_float(v); }
    __device__ static __forceinline__ raw from_f(float f) { return float_to_half_bits(f); }
};
template <> struct St<BF16> {
    typedef uint16_t raw;
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float to_f(raw v) { return bf16_bits_to_float(v); }
    __device__ static __forceinline__ raw from_f(float f) { return float_to_bf16_bits(f); }
};

// OCP 8-bit floats through gfx950's conversion instructions: widening is exact;
// narrowing rounds to nearest even, after a clamp to the largest finite value
// (the instructions would otherwise give NaN for e4m3 and inf for e5m2).
template <> struct St<E4M3> {
    typedef uint8_t raw;
    static constexpr int bytes = 1;
    static constexpr float vmax = 448.f;
    __device__ static __forceinline__ float to_f(raw v) { return __builtin_amdgcn_cvt_f32_fp8((int)v, 0); }
    __device__ static __forceinline__ raw from_f(float f) {
        f = fminf(fmaxf(f, -vmax), vmax);
        return (raw)(__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.f, 0, false) & 0xFF);
    }
};
template <> struct St<E5M2> {
    typedef uint8_t raw;
    static constexpr int bytes = 1;
    static constexpr float vmax = 57344.f;
    __device__ static __forceinline__ float to_f(raw v) { return __builtin_amdgcn_cvt_f32_bf8((int)v, 0); }
    __device__ static __forceinline__ raw from_f(float f) {
        f = fminf(fmaxf(f, -vmax), vmax);
        return (raw)(__builtin_amdgcn_cvt_pk_bf8_f32(f, 0.f, 0, false) & 0xFF);
    }
};

// byte b (a constant after unrolling) of a word of four 8-bit floats, widened
template <int DT>
__device__ __forceinline__ float fp8_byte(uint32_t w, int b) {
    const int x = (int)w;
    if constexpr (DT == E4M3) {
        switch (b & 3) {
            case 0: return __builtin_amdgcn_cvt_f32_fp8(x, 0);
            case 1: return __builtin_amdgcn_cvt_f32_fp8(x, 1);
            case 2: return __builtin_amdgcn_cvt_f32_fp8(x, 2);
            default: return __builtin_amdgcn_cvt_f32_fp8(x, 3);
        }
    } else {
        switch (b & 3) {
            case 0: return __builtin_amdgcn_cvt_f32_bf8(x, 0);
            case 1: return __builtin_amdgcn_cvt_f32_bf8(x, 1);
            case 2: return __builtin_amdgcn_cvt_f32_bf8(x, 2);
            default: return __builtin_amdgcn_cvt_f32_bf8(x, 3);
        }
    }
}

// Load n contiguous storage elements (n * bytes a multiple of 4) and widen.
template <int DT, int N>
__device__ __forceinline__ void load_widen(const void* p, float* out) {
    typedef typename St<DT>::raw R;
    if constexpr (St<DT>::bytes == 4) {
        static_assert(N % 4 == 0, "");
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            float4 v = reinterpret_cast<const float4*>(p)[i];
            out[4 * i + 0] = v.x;
            out[4 * i + 1] = v.y;
            out[4 * i + 2] = v.z;
            out[4 * i + 3] = v.w;
        }
    } else if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            uint4 v = reinterpret_cast<const uint4*>(p)[i];
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[8 * i + 2 * j + 0] = St<DT>::to_f((R)(w[j] & 0xFFFFu));
                out[8 * i + 2 * j + 1] = St<DT>::to_f((R)(w[j] >> 16));
            }
        }
    } else {
        static_assert(N % 4 == 0, "");
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            uint2 v = reinterpret_cast<const uint2*>(p)[i];
            uint32_t w[2] = {v.x, v.y};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                out[4 * i + 2 * j + 0] = St<DT>::to_f((R)(w[j] & 0xFFFFu));
                out[4 * i + 2 * j + 1] = St<DT>::to_f((R)(w[j] >> 16));
            }
        }
    }
}

// N storage elements held as raw 32-bit words (loaded with one or two vector
// loads), widened to fp32 only where they are used.
template <int DT, int N>
struct RawVec {
    static constexpr int words = N * St<DT>::bytes / 4;
    uint32_t w[words];
};

template <int DT, int N>
__device__ __forceinline__ void load_raw(RawVec<DT, N>& r, const void* p) {
    constexpr int W = RawVec<DT, N>::words;
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int i = 0; i < W / 4; ++i) {
            uint4 v = load_stream16(reinterpret_cast<const uint4*>(p) + i);
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    } else {
        static_assert(W % 2 == 0, "");
        typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < W / 2; ++i) {
            const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p) + i);
            r.w[2 * i + 0] = v.x;
            r.w[2 * i + 1] = v.y;
        }
    }
}

template <int DT, int N>
__device__ __forceinline__ float raw_at(const RawVec<DT, N>& r, int i) {
    if constexpr (St<DT>::bytes == 4) {
        return __uint_as_float(r.w[i]);
    } else if constexpr (St<DT>::bytes == 1) {
        return fp8_byte<DT>(r.w[i >> 2], i & 3);
    } else {
        const uint32_t w = r.w[i >> 1];
        return St<DT>::to_f((typename St<DT>::raw)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
    }
}

template <int DT>
__device__ __forceinline__ void store_round(void* base, long idx, float v) {
    reinterpret_cast<typename St<DT>::raw*>(base)[idx] = St<DT>::from_f(v);
}

// One K or V element into the cache: the model's storage type, or an 8-bit float.
template <int DT>
__device__ __forceinline__ void store_kv(void* base, long idx, float v, int kv_dt) {
    if (kv_dt == E4M3) reinterpret_cast<uint8_t*>(base)[idx] = St<E4M3>::from_f(v);
    else if (kv_dt == E5M2) reinterpret_cast<uint8_t*>(base)[idx] = St<E5M2>::from_f(v);
    else store_round<DT>(base, idx, v);
}

template <int DT>
__device__ __forceinline__ float load_one(const void* base, long idx) {
    return St<DT>::to_f(reinterpret_cast<const typename St<DT>::raw*>(base)[idx]);
}

// ---- wave64 shuffles ----------------------------------------------------

// Sum over the 16 lanes of each DPP row (lanes 16r..16r+15); every lane of the
// row receives the row's sum, computed in the same order in every lane.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

// Sum over the 64 lanes of a wave, the same fixed order for every call: pairs,
// quads, half rows and rows through DPP, then the four rows through readlane.
// The result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ int shfl_xor(int v, int mask) { return __shfl_xor(v, mask, kWave); }

}  // namespace vs
