// operands.h -- matrix-instruction operand helpers shared by the GEMM kernels
// (gfx950).  Internal; included by the kernel sources only.
//
// "509 tokens a second of prompt: the Hadamard route ships", section "Why
// prompts are a matrix-unit problem": a Q4_0 code u means u-8, which is the
// code with its top bit flipped read as a 4-bit two's-complement number.
// gfx950 has no int4 matrix instruction, so nibbles are widened to int8 in
// registers as 16 * value (the nibble in the top half of a byte): the
// instruction then returns 256 * S for 4-bit activations (16 * S for 8-bit
// ones), and the power of two is removed once, when the output is stored.
//
// The accumulator input of every matrix instruction is 0x4B400000 (1.5*2^23
// as fp32), so the int32 result read as fp32 is exactly 12582912 + 256*S
// (|256*S| < 2^22); t = fma(F, dw, -12582912*dw) = 256*S*dw exactly (dw is an
// fp16 value, 11 significant bits), then acc = fma(t, da, acc).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bpg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

// Activation nibbles (two's complement) of one dword -> 8 int8 = 16 * value:
// low nibbles first, then high nibbles.
__device__ __forceinline__ uint32_t act_lo(uint32_t d) { return (d << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t act_hi(uint32_t d) { return d & 0xF0F0F0F0u; }
// Q4_0 nibbles u -> top bit flipped (u XOR 8 is u-8 in two's complement) ->
// 16*(u-8).
__device__ __forceinline__ uint32_t q40_lo(uint32_t d) { return ((d << 4) ^ 0x80808080u) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t q40_hi(uint32_t d) { return (d ^ 0x88888888u) & 0xF0F0F0F0u; }

__device__ __forceinline__ long pack2(uint32_t lo, uint32_t hi)
{
    return (long)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t bf16_rne(float v)
{
    const uint32_t u = __float_as_uint(v);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One output element: fp32, or bf16 when the problem asks for it (the
// choice is uniform across the launch).
__device__ __forceinline__ void store_y(const GemmProblem &p, int64_t idx, float v)
{
    if (p.y16)
        p.y16[idx] = bf16_rne(v);
    else
        p.y[idx] = v;
}

// Workgroups are dispatched round-robin over the 8 XCDs (w % 8 selects the
// XCD).  Hand each XCD a contiguous range of logical tiles, so tiles that
// share weight columns share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total)
{
    if (total % 8 != 0)
        return w;
    return (w % 8) * (total / 8) + w / 8;
}

// Direct global -> LDS loads (global_load_lds_*) name their source and
// destination through these address spaces.
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void glb_void;

// An integer the optimizer cannot take apart.  LDS addresses built as
// "array + opaque offset" stay one step from their array, which lets the
// compiler attribute every read to its buffer and so not wait for the direct
// loads into the other buffer before it.
__device__ __forceinline__ uint32_t opaque(uint32_t x)
{
    asm("" : "+v"(x));
    return x;
}

// The same address in every lane, held in scalar registers (a direct load
// then takes it as its scalar base and the lane offset as a 32-bit register).
__device__ __forceinline__ const uint8_t *uniform(const uint8_t *ptr)
{
    const uint64_t a = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}

// Operand and result registers of the two matrix instruction shapes.
template <int MF> struct Mfma;

template <> struct Mfma<16> {
    typedef long Op;
    typedef v4i Acc;
    // lane l: row / column l % 16 of the tile and K group g = l / 16, which
    // holds bytes 4g..4g+3 of the packed block (elements 4g..4g+3 from the
    // low nibbles, 16+4g..16+4g+3 from the high ones); result register r of
    // lane l is row 4g + r, column l % 16.
    static __device__ __forceinline__ int rc(int lane) { return lane & 15; }
    static __device__ __forceinline__ int kg(int lane) { return lane >> 4; }
    static __device__ __forceinline__ int out_row(int g, int r) { return 4 * g + r; }
    static __device__ __forceinline__ Acc mma(Op a, Op b, Acc c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<32> {
    typedef v4i Op;
    typedef v16i Acc;
    // lane l: row / column l % 32 of the tile and K half g = l / 32, which
    // holds bytes 8g..8g+7 of the packed block (elements 8g..8g+7 low,
    // 16+8g..16+8g+7 high); result register r of lane l is row
    // 8 (r / 4) + 4g + r % 4, column l % 32.
    static __device__ __forceinline__ int rc(int lane) { return lane & 31; }
    static __device__ __forceinline__ int kg(int lane) { return lane >> 5; }
    static __device__ __forceinline__ int out_row(int g, int r) { return 8 * (r >> 2) + 4 * g + (r & 3); }
    static __device__ __forceinline__ Acc mma(Op a, Op b, Acc c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
};

} // namespace
} // namespace bpg
