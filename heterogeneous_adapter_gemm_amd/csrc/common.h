// Device helpers shared by the gfx950 kernels: 16-byte vector access,
// bf16 <-> fp32 conversion and the matrix-core (MFMA) step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hagemm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct bf16_t {
    uint16_t bits;
};

template <typename E>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16 bytes
};
template <>
struct Elem<bf16_t> {
    static constexpr int kVec = 8;
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even: gfx950 converts in
// hardware (v_cvt_pk_bf16_f32), NaN stays NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16); }

// unpack a 16-byte vector of E into floats
__device__ __forceinline__ void unpack(const u32x4& v, float (&o)[8], bf16_t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = bf16_lo(v[i]);
        o[2 * i + 1] = bf16_hi(v[i]);
    }
}
__device__ __forceinline__ void unpack(const u32x4& v, float (&o)[4], float) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
}

__device__ __forceinline__ u32x4 pack(const float (&o)[8], bf16_t) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16(o[2 * i], o[2 * i + 1]);
    return r;
}
__device__ __forceinline__ u32x4 pack(const float (&o)[4], float) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(o[i]);
    return r;
}

// One 16-byte-per-lane step of a 16x16 output block on the matrix cores:
// lane l supplies row/column (l % 16) of each operand and the 16 bytes of K
// that lane group (l / 16) holds; both operands must use the same K layout.
// bf16: one v_mfma_f32_16x16x32_bf16; fp32: four v_mfma_f32_16x16x4_f32,
// element e of every lane's vector feeding step e.
__device__ __forceinline__ f32x4 mma_step(const u32x4& a, const u32x4& b, f32x4 c, bf16_t) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}
__device__ __forceinline__ f32x4 mma_step(const u32x4& a, const u32x4& b, f32x4 c, float) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
    return c;
}

// Workgroups are dealt round-robin over the 8 XCDs (workgroup b runs on XCD b % 8).
// xcd_logical numbers them so that consecutive logical ids run on one XCD and share
// its L2: the first ceil(total / 8) ids on XCD 0, and so on.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical(int bid, int total) {
    const int q = total / kXcds, rr = total % kXcds;
    const int xcd = bid % kXcds, idx = bid / kXcds;
    return xcd < rr ? xcd * (q + 1) + idx : rr * (q + 1) + (xcd - rr) * q + idx;
}

typedef __attribute__((address_space(3))) void* lds_vptr;

// buffer resource word 3 for raw (unformatted, unswizzled) 32-bit access on CDNA
constexpr int kRawBufferFlags = 0x00020000;

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N_>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N_ & 0xF) | ((N_ >> 4) << 14) | (0x7 << 4));
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained
template <int N_>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N_ & 0xF) | ((N_ >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane straight into LDS (lane i -> lds + 16 i) by a raw buffer
// load of base (bytes long) at byte offset voff + soff: voff per lane, soff
// uniform.  A non-template function, so the host pass of templates that call
// it never looks the target builtin up.
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, void* lds, int voff, int soff) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds, 16, voff, soff, 0, 0);
}

// 16 bytes per lane straight into LDS (lane i -> lds + 16 i) from a per-lane global address
__device__ __forceinline__ void global_load_lds16(const void* p, void* lds) {
    __builtin_amdgcn_global_load_lds(const_cast<void*>(p), (lds_vptr)lds, 16, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace hagemm
