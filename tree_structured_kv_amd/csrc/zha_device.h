// zha_device.h -- small device helpers shared by the libzha kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace zha {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(bf16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Four consecutive elements as floats (one 16- or 8-byte load).
typedef float gf4_t __attribute__((ext_vector_type(4)));
typedef uint32_t gu4_t __attribute__((ext_vector_type(4)));
typedef uint32_t gu2_t __attribute__((ext_vector_type(2)));
#define ZHA_GLOBAL(T) const __attribute__((address_space(1))) T *

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float *p, float *o) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    // streaming read (nontemporal): data read once and not again soon
    static __device__ __forceinline__ void load_nt(const float *p, float *o) {
        const gf4_t v = __builtin_nontemporal_load((ZHA_GLOBAL(gf4_t))p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct Vec4<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t *p, float *o) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void load_nt(const bf16_t *p, float *o) {
        const gu2_t v = __builtin_nontemporal_load((ZHA_GLOBAL(gu2_t))p);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};

// Loads through pointers known to address device (global) memory.  When a
// pointer is read from a table in LDS the compiler cannot tell its address
// space and emits flat loads, which also count on the LDS counter: a later
// wait for an LDS read then waits for every flat load still in flight.
__device__ __forceinline__ gf4_t gload_f4(const void *p) { return *(ZHA_GLOBAL(gf4_t))p; }
__device__ __forceinline__ gu4_t gload_u4(const void *p) { return *(ZHA_GLOBAL(gu4_t))p; }
__device__ __forceinline__ gu2_t gload_u2(const void *p) { return *(ZHA_GLOBAL(gu2_t))p; }
__device__ __forceinline__ float gload_f(const float *p) { return *(ZHA_GLOBAL(float))p; }
__device__ __forceinline__ gu4_t gload_u4_nt(const void *p) { return __builtin_nontemporal_load((ZHA_GLOBAL(gu4_t))p); }
__device__ __forceinline__ gu2_t gload_u2_nt(const void *p) { return __builtin_nontemporal_load((ZHA_GLOBAL(gu2_t))p); }

// Read-only data at a wavefront-uniform address, through the constant
// address space (scalar loads into SGPRs).  Only for memory that no
// workgroup writes while the kernel runs.
#define ZHA_CONST(T) const __attribute__((address_space(4))) T *
__device__ __forceinline__ float cload_f(const float *p) { return *(ZHA_CONST(float))p; }
__device__ __forceinline__ uint32_t cload_u32(const uint32_t *p) { return *(ZHA_CONST(uint32_t))p; }

// Vec4 through a global pointer.
template <typename T> struct GVec4;
template <> struct GVec4<float> {
    static __device__ __forceinline__ void load(const float *p, float *o) {
        const gf4_t v = gload_f4(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct GVec4<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t *p, float *o) {
        const gu2_t v = gload_u2(p);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};

// 16 bytes of a row as floats: 4 fp32 or 8 bf16 elements.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float *p, float (&o)[4]) {
        float4 v = *reinterpret_cast<const float4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ void load_nt(const float *p, float (&o)[4]) {
        const gf4_t v = __builtin_nontemporal_load((ZHA_GLOBAL(gf4_t))p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const bf16_t *p, float (&o)[8]) {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load_nt(const bf16_t *p, float (&o)[8]) {
        const gu4_t v = __builtin_nontemporal_load((ZHA_GLOBAL(gu4_t))p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(v[i] << 16);
            o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
};

// DPP cross-lane moves (gfx9 encodings): quad_perm xor 1 / xor 2, and the
// 8- and 16-lane mirrors, which pair the two halves of a group once the
// values are uniform inside each half.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// Sum over aligned groups of WIDTH lanes (WIDTH in {16, 32}); every lane of
// a group gets the group's sum.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    if (WIDTH == 32)   // swap the two 16-lane rows of each 32-lane half
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    return v;
}

// Max over aligned groups of WIDTH consecutive lanes (WIDTH in {1, 2, 4, 8,
// 16}); every lane of a group gets the group's max.
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
    if (WIDTH >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
    if (WIDTH >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
    if (WIDTH >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if (WIDTH >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    return v;
}

// Lane exchanges without the LDS permute unit.  xor_lane<J>: the value of
// lane (lane ^ J) for J a power of two below 64: within a row of 16 lanes by
// DPP (quad_perm for 1 and 2, row shifts for 4, row rotate for 8), across
// rows by gfx950's row swaps (v_permlane16_swap / v_permlane32_swap, each
// called with the value in both operands: the swapped halves are the
// partner's).  wave_scan_u64: inclusive sum over the 64 lanes by DPP row
// shifts and the row broadcasts of lanes 15 and 31.
constexpr int kDppShl4 = 0x104;       // row_shl:4: lane i reads lane i+4 of its row
constexpr int kDppShr = 0x110;        // row_shr:N (0x110 + N): lane i reads lane i-N of its row
constexpr int kDppRor8 = 0x128;       // row_ror:8: lane i reads lane i^8 of its row
constexpr int kDppBcast15 = 0x142;    // lane 15 of each row to the next row
constexpr int kDppBcast31 = 0x143;    // lane 31 to rows 2 and 3

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xf, false));
}

template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    const int lane = __lane_id();
    if constexpr (J == 1) {
        return dpp_u32<kDppXor1>(v);
    } else if constexpr (J == 2) {
        return dpp_u32<kDppXor2>(v);
    } else if constexpr (J == 4) {
        const uint32_t up = dpp_u32<kDppShl4>(v), dn = dpp_u32<kDppShr + 4>(v);
        return (lane & 4) ? dn : up;
    } else if constexpr (J == 8) {
        return dpp_u32<kDppRor8>(v);
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(J == 32, "xor_lane: J is a power of two below 64");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

template <int J>
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long v) {
    const uint32_t lo = xor_lane<J>(static_cast<uint32_t>(v));
    const uint32_t hi = xor_lane<J>(static_cast<uint32_t>(v >> 32));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const uint32_t lo = dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(v));
    const uint32_t hi = dpp_u32<CTRL, ROWS>(static_cast<uint32_t>(v >> 32));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x) {
    x += dpp_u64<kDppShr + 1>(x);
    x += dpp_u64<kDppShr + 2>(x);
    x += dpp_u64<kDppShr + 4>(x);
    x += dpp_u64<kDppShr + 8>(x);
    x += dpp_u64<kDppBcast15, 0xa>(x);
    x += dpp_u64<kDppBcast31, 0xc>(x);
    return x;
}

__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
    x += dpp_u32<kDppShr + 1>(x);
    x += dpp_u32<kDppShr + 2>(x);
    x += dpp_u32<kDppShr + 4>(x);
    x += dpp_u32<kDppShr + 8>(x);
    x += dpp_u32<kDppBcast15, 0xa>(x);
    x += dpp_u32<kDppBcast31, 0xc>(x);
    return x;
}

// Lane l's 64-bit value for every lane (l wavefront-uniform).
__device__ __forceinline__ unsigned long long read_lane64(unsigned long long v, int l) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// The sum over all 64 lanes, in every lane.
__device__ __forceinline__ unsigned long long wave_total_u64(unsigned long long v) {
    return read_lane64(wave_scan_u64(v), 63);
}

__device__ __forceinline__ uint32_t wave_total_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_scan_u32(v)), 63));
}

// xor_lane with the distance a (power-of-two) value that unrolled loops fold.
__device__ __forceinline__ uint32_t xor_lane_n(uint32_t v, int j) {
    switch (j) {
        case 1: return xor_lane<1>(v);
        case 2: return xor_lane<2>(v);
        case 4: return xor_lane<4>(v);
        case 8: return xor_lane<8>(v);
        case 16: return xor_lane<16>(v);
        default: return xor_lane<32>(v);
    }
}
__device__ __forceinline__ float xor_lane_f(float v, int j) { return __uint_as_float(xor_lane_n(__float_as_uint(v), j)); }
__device__ __forceinline__ unsigned long long xor_lane64_n(unsigned long long v, int j) {
    const uint32_t lo = xor_lane_n(static_cast<uint32_t>(v), j);
    const uint32_t hi = xor_lane_n(static_cast<uint32_t>(v >> 32), j);
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Butterfly sum / max over aligned groups of `width` lanes (every lane of a
// group gets the result; partners exactly as a lane-xor shuffle gives them).
__device__ __forceinline__ float wave_sum(float v, int width) {
#pragma unroll
    for (int off = 1; off < width; off <<= 1) v += xor_lane_f(v, off);
    return v;
}

__device__ __forceinline__ float wave_max(float v, int from, int to) {
#pragma unroll
    for (int off = from; off < to; off <<= 1) v = fmaxf(v, xor_lane_f(v, off));
    return v;
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The (sequence, KV head) pair a walk reads: walks are laid out as
// [batch][query head][query], and query head h uses KV head h / group.
__device__ __forceinline__ int64_t walk_pair(int64_t w, int qph, int heads, int group, int kv_heads) {
    const int64_t hq = w / qph;
    const int64_t b = hq / heads;
    const int h = static_cast<int>(hq % heads);
    return b * kv_heads + h / group;
}

// XCD-aware workgroup order: the hardware hands consecutive workgroup ids to
// the 8 XCDs in turn; remap so each XCD gets one contiguous range of logical
// ids (neighbouring walks share tree nodes in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
    if ((nb & 7) != 0) return bid;
    int per = nb >> 3;
    return (bid & 7) * per + (bid >> 3);
}

}  // namespace zha
