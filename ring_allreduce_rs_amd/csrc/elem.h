// elem.h -- device-side element arithmetic of one ring hop (gfx950).
//
// A hop combines the partial result travelling round the ring with the
// receiving rank's own element.  The pages name the reduction (sum, max) and
// the DDP average (sum, then divide by the world size: "Allreduce：大模型分布式
// 训练的核心通信算法与优化实践", sections 3.1-3.2) but not its arithmetic; the
// rules implemented here are:
//   int32 SUM  two's-complement wrap-around add
//   fp32  SUM  one binary32 add, round to nearest even (no contraction, no
//              wider accumulator, subnormals kept)
//   bf16  SUM  widen both to fp32, add in fp32, round the sum to bf16
//              (nearest even) -- every hop rounds
//   MAX        IEEE-754-2019 maximum: NaN wins (canonical quiet NaN), +0 > -0
//   AVG        finished SUM divided once by N: fp32 correctly rounded
//              division; bf16 rounds the fp32 quotient
//
// Storage is handled as raw 32-bit words so one 16-byte load feeds 4 fp32 /
// int32 lanes or 8 bf16 lanes.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arlib {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// IEEE-754-2019 maximum of two binary32 bit patterns.  Equal values differ at
// most in the sign of a zero; AND-ing the patterns gives -0 only if both are -0.
__device__ __forceinline__ uint32_t fmaximum_bits(uint32_t a, uint32_t b) {
    const float fa = as_f32(a), fb = as_f32(b);
    if (fa != fa || fb != fb) return 0x7fc00000u;
    if (fa == fb) return a & b;
    return fa > fb ? a : b;
}

// binary32 -> bf16, round to nearest, ties to even; NaN -> canonical quiet
// NaN 0x7FC0.  gfx950 converts with v_cvt_pk_bf16_f32 (two values per
// instruction).  Its result was compared on MI355X with the integer rule --
// add 0x7FFF plus the lowest kept bit, drop 16 bits -- for all 2^32 fp32 bit
// patterns: identical for every non-NaN input (subnormals, overflow by
// rounding and ties included); NaN inputs keep their sign and payload there,
// so they are replaced by 0x7FC0 here.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)f);
    return f != f ? 0x7fc0u : h;
}

// Two values rounded at once: lo into bits 0..15, hi into bits 16..31.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    if (lo != lo) r = (r & 0xffff0000u) | 0x7fc0u;
    if (hi != hi) r = (r & 0x0000ffffu) | 0x7fc00000u;
    return r;
}

__device__ __forceinline__ float bf16_widen(uint32_t h) { return as_f32(h << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f32(w & 0xffff0000u); }

// x / n, correctly rounded.  When n is a power of two the caller passes
// inv = 1/n (exact); x * 2^-k and x / 2^k are then the same real number
// rounded once, so the product is the correctly rounded quotient, subnormal
// results included (denormals are not flushed).  Otherwise inv is 0 and the
// IEEE division is used.
__device__ __forceinline__ float div_by_n(float x, float nf, float inv) {
    return inv != 0.0f ? __fmul_rn(x, inv) : __fdiv_rn(x, nf);
}

// Every op exposes: element size, one-element combine/finish on the low bits
// of a word, and whole-word combine/finish (two bf16 per word).
struct OpI32Sum {
    static constexpr int kElemBytes = 4;
    __device__ static uint32_t comb_elem(uint32_t a, uint32_t b) { return a + b; }
    __device__ static uint32_t finish_elem(uint32_t a, float, float) { return a; }
    __device__ static uint32_t comb_word(uint32_t a, uint32_t b) { return a + b; }
    __device__ static uint32_t finish_word(uint32_t a, float, float) { return a; }
};

struct OpI32Max {
    static constexpr int kElemBytes = 4;
    __device__ static uint32_t comb_elem(uint32_t a, uint32_t b) {
        return (int32_t)a > (int32_t)b ? a : b;
    }
    __device__ static uint32_t finish_elem(uint32_t a, float, float) { return a; }
    __device__ static uint32_t comb_word(uint32_t a, uint32_t b) { return comb_elem(a, b); }
    __device__ static uint32_t finish_word(uint32_t a, float, float) { return a; }
};

struct OpF32Sum {
    static constexpr int kElemBytes = 4;
    __device__ static uint32_t comb_elem(uint32_t a, uint32_t b) {
        return as_u32(__fadd_rn(as_f32(a), as_f32(b)));
    }
    __device__ static uint32_t finish_elem(uint32_t a, float nf, float inv) {
        return as_u32(div_by_n(as_f32(a), nf, inv));
    }
    __device__ static uint32_t comb_word(uint32_t a, uint32_t b) { return comb_elem(a, b); }
    __device__ static uint32_t finish_word(uint32_t a, float nf, float inv) {
        return finish_elem(a, nf, inv);
    }
};

struct OpF32Max {
    static constexpr int kElemBytes = 4;
    __device__ static uint32_t comb_elem(uint32_t a, uint32_t b) { return fmaximum_bits(a, b); }
    __device__ static uint32_t finish_elem(uint32_t a, float, float) { return a; }
    __device__ static uint32_t comb_word(uint32_t a, uint32_t b) { return fmaximum_bits(a, b); }
    __device__ static uint32_t finish_word(uint32_t a, float, float) { return a; }
    // A fold kept in registers takes the hardware's IEEE-754-2019 maximum (a
    // NaN if either operand is one, -0 below +0; gfx950 issues it as
    // v_maximum3_f32, two hops per instruction) and makes a NaN canonical
    // once, at the end.  A maximum is one of its operands and does not depend
    // on the order of the fold, so the bits are those of the rule above
    // applied hop by hop.
    __device__ static uint32_t fold_word(uint32_t a, uint32_t b) {
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(as_f32(a), as_f32(b)));
    }
    __device__ static uint32_t canon_word(uint32_t a) {
        return as_f32(a) != as_f32(a) ? 0x7fc00000u : a;
    }
};

struct OpBF16Sum {
    static constexpr int kElemBytes = 2;
    __device__ static uint32_t comb_elem(uint32_t a, uint32_t b) {
        return bf16_rne(__fadd_rn(bf16_widen(a & 0xffffu), bf16_widen(b & 0xffffu)));
    }
    __device__ static uint32_t finish_elem(uint32_t a, float nf, float inv) {
        return bf16_rne(div_by_n(bf16_widen(a & 0xffffu), nf, inv));
    }
    __device__ static uint32_t comb_word(uint32_t a, uint32_t b) {
        return bf16x2_rne(__fadd_rn(bf16_lo(a), bf16_lo(b)), __fadd_rn(bf16_hi(a), bf16_hi(b)));
    }
    __device__ static uint32_t finish_word(uint32_t a, float nf, float inv) {
        return bf16x2_rne(div_by_n(bf16_lo(a), nf, inv), div_by_n(bf16_hi(a), nf, inv));
    }
};

struct OpBF16Max {
    static constexpr int kElemBytes = 2;
    // the maximum of two bf16 values is one of them, so it needs no rounding
    __device__ static uint32_t comb_elem(uint32_t a, uint32_t b) {
        const uint32_t m = fmaximum_bits((a & 0xffffu) << 16, (b & 0xffffu) << 16);
        return m >> 16;
    }
    __device__ static uint32_t finish_elem(uint32_t a, float, float) { return a & 0xffffu; }
    __device__ static uint32_t comb_word(uint32_t a, uint32_t b) {
        return comb_elem(a, b) | (comb_elem(a >> 16, b >> 16) << 16);
    }
    __device__ static uint32_t finish_word(uint32_t a, float, float) { return a; }
};

// Copy-only "op" for the AllGather paths (element size matters, values do not).
template <int EB>
struct OpCopy {
    static constexpr int kElemBytes = EB;
};

// ---------------------------------------------------------------- memory units
//
// A Unit is what one lane moves per access: 16 bytes on the vector path, one
// element on the scalar path (used for the unaligned head and tail of a chunk,
// and for buffers whose addresses disagree modulo 16).

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}

template <int EB>
__device__ __forceinline__ uint32_t ld_elem(const void* p) {
    if constexpr (EB == 4) return *reinterpret_cast<const uint32_t*>(p);
    else return *reinterpret_cast<const uint16_t*>(p);
}

template <int EB>
__device__ __forceinline__ void st_elem(void* p, uint32_t v) {
    if constexpr (EB == 4) *reinterpret_cast<uint32_t*>(p) = v;
    else *reinterpret_cast<uint16_t*>(p) = (uint16_t)v;
}

template <class Op>
__device__ __forceinline__ u32x4 comb4(u32x4 a, u32x4 b) {
    u32x4 r;
    r.x = Op::comb_word(a.x, b.x);
    r.y = Op::comb_word(a.y, b.y);
    r.z = Op::comb_word(a.z, b.z);
    r.w = Op::comb_word(a.w, b.w);
    return r;
}

// Ops with a fold_word: an in-register fold uses it and ends with canon_word
// (see OpF32Max); the others fold with comb_word.
template <class Op, class = void>
struct LazyFold : std::false_type {};
template <class Op>
struct LazyFold<Op, std::void_t<decltype(&Op::fold_word)>> : std::true_type {};

template <class Op>
__device__ __forceinline__ u32x4 fold4(u32x4 a, u32x4 b) {
    u32x4 r;
    r.x = Op::fold_word(a.x, b.x);
    r.y = Op::fold_word(a.y, b.y);
    r.z = Op::fold_word(a.z, b.z);
    r.w = Op::fold_word(a.w, b.w);
    return r;
}

template <class Op>
__device__ __forceinline__ u32x4 canon4(u32x4 a) {
    u32x4 r;
    r.x = Op::canon_word(a.x);
    r.y = Op::canon_word(a.y);
    r.z = Op::canon_word(a.z);
    r.w = Op::canon_word(a.w);
    return r;
}

template <class Op>
__device__ __forceinline__ u32x4 finish4(u32x4 a, float nf, float inv) {
    u32x4 r;
    r.x = Op::finish_word(a.x, nf, inv);
    r.y = Op::finish_word(a.y, nf, inv);
    r.z = Op::finish_word(a.z, nf, inv);
    r.w = Op::finish_word(a.w, nf, inv);
    return r;
}

}  // namespace arlib
