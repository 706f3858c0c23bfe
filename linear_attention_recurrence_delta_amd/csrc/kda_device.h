// kda_device.h -- device-side building blocks shared by the KDA kernels
// (gfx950 / CDNA4 only): bf16 storage helpers and 16x16 MFMA wrappers.
//
// K-index convention.  Every 16x16 matrix product here works on "K blocks"
// of 16.  Inside block kb, lane l of a wave (g = l / 16, i = l % 16) supplies
// the four logical k values 16*kb + 4*g + p, p = 0..3, for operand row i of A
// (A[i][k]) and for operand column i of B (B[k][i]).  The accumulator layout
// of a 16x16 MFMA puts C[4*g + p][i] in lane l, register p -- the same
// (g, p) -> index map.  So the output of one product, taken as rows, is
// already a B operand of the next product over those rows, with no data
// movement.  The hardware's own k order inside an instruction does not
// matter: A and B are fed through the same (lane, slot) -> k map, and the
// product sums over all k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// bf16 values are stored as raw 16-bit patterns.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
// acc + lo(a) lo(b) + hi(a) hi(b) for two packed bf16 pairs (v_dot2c_f32_bf16:
// products exact, fp32 sum).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ---------------------------------------------------------------------------
// Element traits: load/store of scalars and of the 4-value operand fragment.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<float> {
    typedef float4 frag;  // four fp32 operand values
    static constexpr int pad = 4;  // LDS row padding in elements (16 bytes)
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static float to_f32(float x) { return x; }
    __device__ __forceinline__ static float from_f32(float x) { return x; }
    __device__ __forceinline__ static frag make(float a, float b, float c, float d) {
        return make_float4(a, b, c, d);
    }
    __device__ __forceinline__ static frag make(f32x4 v) { return make_float4(v[0], v[1], v[2], v[3]); }
    __device__ __forceinline__ static float get(const frag& f, int p) {
        return p == 0 ? f.x : p == 1 ? f.y : p == 2 ? f.z : f.w;
    }
    __device__ __forceinline__ static frag zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

template <> struct Elem<bf16_t> {
    typedef uint2 frag;  // four bf16 operand values, two per dword
    static constexpr int pad = 8;  // LDS row padding in elements (16 bytes)
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
    __device__ __forceinline__ static float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
    __device__ __forceinline__ static bf16_t from_f32(float x) { bf16_t r; r.bits = f32_to_bf16(x); return r; }
    __device__ __forceinline__ static frag make(float a, float b, float c, float d) {
        return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
    }
    __device__ __forceinline__ static frag make(f32x4 v) { return make(v[0], v[1], v[2], v[3]); }
    __device__ __forceinline__ static float get(const frag& f, int p) {
        const uint32_t w = (p < 2) ? f.x : f.y;
        return __uint_as_float((p & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ static frag zero() { return make_uint2(0u, 0u); }
};

// Read / write a 4-value fragment at an LDS (or global) address.  Addresses
// are 8-byte (bf16) or 16-byte (fp32) aligned by construction of the layouts.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag ld_frag(const T* p) {
    return *reinterpret_cast<const typename Elem<T>::frag*>(p);
}
template <typename T>
__device__ __forceinline__ void st_frag(T* p, const typename Elem<T>::frag& f) {
    *reinterpret_cast<typename Elem<T>::frag*>(p) = f;
}

// ---------------------------------------------------------------------------
// 16x16 products with fp32 accumulation.
//   mma16: one K block (16).      mma32: two K blocks (32).
//
// An accumulator chain stays within one instruction shape.  A bf16 16x16x16
// product that takes the result of a 16x16x32 product as its accumulator
// input a few instructions later read part of it before it was written
// (some lanes and registers kept the older value): the compiler inserts no
// wait there, as it does for a chain of one shape.  Products of different
// shapes go to separate accumulators and are added with VALU.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma16(f32x4& acc, const float4& a, const float4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const uint2& a, const uint2& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x4& acc, const float4& a0, const float4& a1,
                                      const float4& b0, const float4& b1) {
    mma16(acc, a0, b0);
    mma16(acc, a1, b1);
}
__device__ __forceinline__ void mma32(f32x4& acc, const uint2& a0, const uint2& a1,
                                      const uint2& b0, const uint2& b1) {
    const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
    const uint4 b = make_uint4(b0.x, b0.y, b1.x, b1.y);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Raw buffer resource over `bytes` bytes from `base` (stride 0; accesses past
// `bytes` read zeros and drop stores).  Store data taken from an element of an
// ext-vector goes through __float_as_uint: __builtin_bit_cast of such an
// element (v[i] as an lvalue) compiled to element 0 for every i.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16r..16r+15):
// lane l ends with x[16r] + ... + x[l].  Each step adds the value of the lane
// n places lower in the row (DPP row_shr:n); lanes with no such lane add 0.
template <int CTRL>
__device__ __forceinline__ float dpp_row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_inclusive_sum16(float x) {
    x += dpp_row_shr<0x111>(x);  // row_shr:1
    x += dpp_row_shr<0x112>(x);  // row_shr:2
    x += dpp_row_shr<0x114>(x);  // row_shr:4
    x += dpp_row_shr<0x118>(x);  // row_shr:8
    return x;
}

// 0 in a VGPR that the compiler cannot fold.  A wave-uniform LDS base plus
// this value stays in one VGPR, so a run of reads at constant distances from
// it is addressed by instruction offsets instead of one copied address
// register per read.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

}  // namespace kda
