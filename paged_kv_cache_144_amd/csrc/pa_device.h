// Device helpers for the CDNA4 (gfx950) kernels: 16-byte lane loads, element conversions,
// wavefront-64 DPP reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Cache dtypes (the values of pa_dtype).  DT_Q8F16 / DT_Q8BF16: one-byte codes with one
// fp16 scale per 32 values; queries and new rows in fp16 / bf16.
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_Q8F16 = 3, DT_Q8BF16 = 4 };

template <int DT>
struct Elem {
    static constexpr int bytes = DT == DT_F32 ? 4 : 2;
    static constexpr int per16 = 16 / bytes;  // elements in one 16-byte lane load
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load of data read once (KV tiles): marked non-temporal so it does not displace
// reused lines in the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Narrower streaming loads for 8-bit tiles: 8 bytes of codes, one 2-byte scale.
__device__ __forceinline__ u32x2 ld8_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ uint32_t ld2_stream(const void* p) {
    return (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Raw buffer resource over `bytes` bytes from p (its address must be wave-uniform).  A lane
// whose offset lies at or past `bytes` reads zeros and its load touches no memory, so with
// bytes = 0 a tile load is issued, counted and discarded without any traffic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
// 16, 8, 4 or 2 bytes at byte offset off of r, non-temporal like ld16_stream
__device__ __forceinline__ u32x4 ld16_buf(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ u32x2 ld8_buf(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
}
__device__ __forceinline__ uint32_t ld4_buf(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2);
}
__device__ __forceinline__ uint32_t ld2_buf(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 2);
}

// ---- element conversion ----------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    return (float)h.x;
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    return (float)h.y;
}

// Widen the elements of one 16-byte load to fp32 (per16 values).
template <int DT>
__device__ __forceinline__ void widen16(u32x4 v, float* f) {
    if constexpr (DT == DT_F32) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    } else if constexpr (DT == DT_F16) {
        f[0] = f16_lo(v.x); f[1] = f16_hi(v.x); f[2] = f16_lo(v.y); f[3] = f16_hi(v.y);
        f[4] = f16_lo(v.z); f[5] = f16_hi(v.z); f[6] = f16_lo(v.w); f[7] = f16_hi(v.w);
    } else {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
}

// fp32 -> bf16 bits, round to nearest even (quiet NaN kept).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two packed 16-bit values of type DT (one v_cvt_pk_{bf16,f16}_f32,
// round to nearest even).
template <int DT>
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    const f32x2 v = {a, b};
    if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
    if constexpr (DT == DT_BF16) return bf16_lo(w);
    else return f16_lo(w);
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
    if constexpr (DT == DT_BF16) return bf16_hi(w);
    else return f16_hi(w);
}

// A probability as the sum of two 16-bit numbers: hi = round(p), lo = round(p - hi).  Two
// matrix products with hi and lo carry p to about 16 significant bits; one 16-bit p alone
// (2^-9 relative for bf16) would put up to ~1e-2 absolute error on rows that see only a
// few tokens.
template <int DT>
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = cvt2<DT>(a, b);
    lo = cvt2<DT>(a - lo16<DT>(hi), b - hi16<DT>(hi));
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Partial dot product of the 16 bytes of q and k held by this lane.
// For 16-bit types q is kept packed (two elements per dword) and the packed dot2
// instructions accumulate in fp32; for fp32 it is a chain of FMAs.
// The vector's components are copied to scalars first: a bit-cast applied directly to a
// component of an ext_vector value is not safe with this compiler (it read component 0).
template <int DT>
__device__ __forceinline__ float dot16(const uint32_t* q, u32x4 k) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    if constexpr (DT == DT_F32) {
        float s = __uint_as_float(q[0]) * __uint_as_float(kw[0]);
        s = fmaf(__uint_as_float(q[1]), __uint_as_float(kw[1]), s);
        s = fmaf(__uint_as_float(q[2]), __uint_as_float(kw[2]), s);
        s = fmaf(__uint_as_float(q[3]), __uint_as_float(kw[3]), s);
        return s;
    } else if constexpr (DT == DT_F16) {
        float s = __builtin_amdgcn_fdot2(as_f16x2(q[0]), as_f16x2(kw[0]), 0.f, false);
        s = __builtin_amdgcn_fdot2(as_f16x2(q[1]), as_f16x2(kw[1]), s, false);
        s = __builtin_amdgcn_fdot2(as_f16x2(q[2]), as_f16x2(kw[2]), s, false);
        s = __builtin_amdgcn_fdot2(as_f16x2(q[3]), as_f16x2(kw[3]), s, false);
        return s;
    } else {
        float s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[0]), as_bf16x2(kw[0]), 0.f, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[1]), as_bf16x2(kw[1]), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[2]), as_bf16x2(kw[2]), s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[3]), as_bf16x2(kw[3]), s, false);
        return s;
    }
}

// ---- cross-lane --------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // reverse within each 8-lane half row
constexpr int DPP_MIRROR = 0x140;       // reverse within each 16-lane row

// Sum over each aligned group of N lanes (N = 4, 8, 16, 32, 64); every lane gets its
// group's sum.  Inside a 16-lane row this is DPP only.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    x += dpp<DPP_XOR1>(x);
    x += dpp<DPP_XOR2>(x);
    if constexpr (N >= 8) x += dpp<DPP_HALF_MIRROR>(x);
    if constexpr (N >= 16) x += dpp<DPP_MIRROR>(x);
    if constexpr (N >= 32)
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // xor 16
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Reductions over the whole wavefront (every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<DPP_XOR1>(x));
    x = fmaxf(x, dpp<DPP_XOR2>(x));
    x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
    x = fmaxf(x, dpp<DPP_MIRROR>(x));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// A read through the constant address space: with a wave-uniform address it becomes a
// scalar load, counted apart from the vector memory operations.  (Vector loads and stores
// share one in-order counter: waiting for a vector load whose value is needed at once means
// waiting for every vector load and store issued before it, tiles in flight included.)
// Only for data that no launch in flight writes.
template <class T>
__device__ __forceinline__ T ld_scalar(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}
// the same, for an address the compiler may hold in vector registers (made uniform first)
template <class T>
__device__ __forceinline__ T ld_scalar_at(const T* p) {
    const uint64_t v = (uint64_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ld_scalar((const T*)(lo | hi << 32));
}

}  // namespace pa
