// quantize.hip -- FWHT-32 fused into per-block activation quantization (gfx950).
//
// "509 tokens a second of prompt: the Hadamard route ships", section "The
// rotation": each 32-value block of activations is rotated by a 32-point
// Walsh-Hadamard transform inside the quantize step, then rounded to 4-bit
// codes sharing one scale.  The pages' RDNA design (two in-thread butterfly
// steps plus three lane shuffles, wave32) is prior art; on CDNA4 (wave64) one
// quad of lanes owns a block:
//
//   lane t of the quad holds elements {4t..4t+3} and {16+4t..16+4t+3};
//   stage h=1 and h=2 pair elements inside each group of four (in-thread),
//   stage h=4 pairs lane t with t^1 and h=8 pairs t with t^2 (DPP quad_perm),
//   stage h=16 pairs element i with i+16 (in-thread, same lane).
// The stage order is 1,2,4,8,16 and every stage gives the lower index a+b and
// the upper a-b, each one fp32 rounding; then every value is multiplied by
// fp32(1/sqrt(32)).  The block scale is amax/7 (8-bit route: amax/127) by
// IEEE division and the code is rint(v/d) with ties to even, clamped; a
// scale of 0 (an all-zero block, or amax/7 underflowing) gives codes 0.
//
// Longer rotations ("Qwen3.8-27B at 45.7 tok/s: DFlash2 in 1bit serve, and
// 4-bit activations with a Hadamard rotation", section "What's next": larger
// rotations spread outliers further): with a span of 64 (128) values the two
// (four) 32-blocks of a span sit in adjacent quads of one wave; stage h=32
// pairs lane l with l^4 and h=64 pairs l with l^8 (ds_swizzle in XOR mode),
// after the five stages of each block, and the factor is fp32(1/sqrt(span)).
// The 32-value scale blocks are unchanged.
//
// This file must be compiled with -ffp-contract=off: no operation above may be
// fused into an FMA, so that the codes are bit-identical to a plain
// step-by-step evaluation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bpg {

namespace {

constexpr int kThreads = 256;           // 64 blocks of 32 values per workgroup
constexpr int kQuantRounds = 1;         // rounds of 16 blocks per wave (more rounds measured slower)
constexpr int kQuadXor1 = 0xB1;         // DPP quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;         // DPP quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float quad_swap(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// One butterfly stage across lanes: the lane whose `upper` flag is set holds
// the upper element b and gets partner - own = a - b; the lower lane gets
// own + partner = a + b.  Negation by flipping the sign bit is exact, so
// partner + (-own) is the IEEE a - b.
template <int CTRL>
__device__ __forceinline__ void cross_stage(float (&v)[8], bool upper)
{
    const uint32_t flip = upper ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float p = quad_swap<CTRL>(v[i]);
        v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ flip);
    }
}

// The same across the quads of a span: lane l pairs with l ^ (PATTERN's XOR
// mask); ds_swizzle bit mode, and mask 0x1F, XOR mask in bits 14:10.
template <int PATTERN>
__device__ __forceinline__ void cross_quad_stage(float (&v)[8], bool upper)
{
    const uint32_t flip = upper ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[i]), PATTERN));
        v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ flip);
    }
}
constexpr int kSwzXor4 = (4 << 10) | 0x1F;
constexpr int kSwzXor8 = (8 << 10) | 0x1F;

__device__ __forceinline__ void load8(const float *src, int t, float (&v)[8])
{
    float4 lo = *reinterpret_cast<const float4 *>(src + 4 * t);
    float4 hi = *reinterpret_cast<const float4 *>(src + 16 + 4 * t);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ void load8(const uint16_t *src, int t, float (&v)[8])
{
    uint2 lo = *reinterpret_cast<const uint2 *>(src + 4 * t);
    uint2 hi = *reinterpret_cast<const uint2 *>(src + 16 + 4 * t);
    v[0] = bf16_to_f32(lo.x & 0xFFFFu); v[1] = bf16_to_f32(lo.x >> 16);
    v[2] = bf16_to_f32(lo.y & 0xFFFFu); v[3] = bf16_to_f32(lo.y >> 16);
    v[4] = bf16_to_f32(hi.x & 0xFFFFu); v[5] = bf16_to_f32(hi.x >> 16);
    v[6] = bf16_to_f32(hi.y & 0xFFFFu); v[7] = bf16_to_f32(hi.y >> 16);
}

// Rotate and quantize one block whose 8 values (this lane's share) are in v.
// rot: 0 (no rotation), 32, 64 or 128 (span of the rotation).
template <int BITS>
__device__ __forceinline__ void quantize_block(float (&v)[8], int t, int rot, int64_t row,
                                               int64_t b, int64_t k, int64_t nb,
                                               uint8_t *__restrict__ codes,
                                               float *__restrict__ scales)
{
    if (rot) {
        // h = 1: pairs (4t, 4t+1), (4t+2, 4t+3) and the same in the upper half
#pragma unroll
        for (int base = 0; base < 8; base += 4) {
            float a0 = v[base], a1 = v[base + 1], a2 = v[base + 2], a3 = v[base + 3];
            v[base] = a0 + a1; v[base + 1] = a0 - a1;
            v[base + 2] = a2 + a3; v[base + 3] = a2 - a3;
        }
        // h = 2: pairs (4t, 4t+2), (4t+1, 4t+3)
#pragma unroll
        for (int base = 0; base < 8; base += 4) {
            float a0 = v[base], a1 = v[base + 1], a2 = v[base + 2], a3 = v[base + 3];
            v[base] = a0 + a2; v[base + 2] = a0 - a2;
            v[base + 1] = a1 + a3; v[base + 3] = a1 - a3;
        }
        // h = 4: element 4t+i pairs with 4(t^1)+i; the even lane is lower
        cross_stage<kQuadXor1>(v, (t & 1) != 0);
        // h = 8: lane t pairs with t^2; lanes 0,1 are lower
        cross_stage<kQuadXor2>(v, (t & 2) != 0);
        // h = 16: element j (v[i]) pairs with j+16 (v[i+4]) in the same lane
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float a = v[i], c = v[i + 4];
            v[i] = a + c;
            v[i + 4] = a - c;
        }
        // h = 32, 64: the blocks of a longer span, in adjacent quads
        const int lane = threadIdx.x & 63;
        if (rot >= 64)
            cross_quad_stage<kSwzXor4>(v, (lane & 4) != 0);
        if (rot >= 128)
            cross_quad_stage<kSwzXor8>(v, (lane & 8) != 0);
        // fp32 nearest to 1/sqrt(rot): 1/sqrt(32), 1/8 and half of 1/sqrt(32)
        const float c = rot == 64 ? 0.125f
                                  : __uint_as_float(rot == 128 ? 0x3DB504F3u : 0x3E3504F3u);
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = v[i] * c;
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
        amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, quad_swap<kQuadXor1>(amax));
    amax = fmaxf(amax, quad_swap<kQuadXor2>(amax));

    constexpr float kQmax = BITS == 4 ? 7.0f : 127.0f;
    constexpr float kQmin = BITS == 4 ? -8.0f : -127.0f;
    // a scale of 0 (an all-zero block, or amax / kQmax underflowing) gives
    // codes 0: every code of such a block dequantizes to 0
    const float d = amax / kQmax;
    // q = rint(v / d) with the IEEE quotient.  The quotient is first taken as
    // v * rcp(d): its error is below |v/d| * 3 * 2^-24 <= 2.3e-5 (|v/d| <= 127),
    // so wherever that product lies at least 1e-4 from a half-integer it
    // rounds to the same integer as the correctly rounded quotient.  Within
    // that band (rare) and for tiny scales the IEEE division decides.
    const bool fast = d >= 0x1p-100f;
    const float rd = __builtin_amdgcn_rcpf(d);
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float r = 0.0f;
        if (d != 0.0f) {
            r = v[i] * rd;
            if (!fast || fabsf(fabsf(r - rintf(r)) - 0.5f) < 1e-4f)
                r = v[i] / d;
            r = rintf(r);
        }
        r = fminf(fmaxf(r, kQmin), kQmax);
        q[i] = (int)r;
    }

    if (BITS == 4) {
        // byte 4t+i = code(4t+i) low nibble | code(16+4t+i) high nibble
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; i++)
            word |= (uint32_t)((q[i] & 0xF) | ((q[i + 4] & 0xF) << 4)) << (8 * i);
        *reinterpret_cast<uint32_t *>(codes + row * (k / 2) + b * 16 + 4 * t) = word;
    } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            lo |= (uint32_t)(q[i] & 0xFF) << (8 * i);
            hi |= (uint32_t)(q[i + 4] & 0xFF) << (8 * i);
        }
        uint8_t *dst = codes + row * k + b * 32;
        *reinterpret_cast<uint32_t *>(dst + 4 * t) = lo;
        *reinterpret_cast<uint32_t *>(dst + 16 + 4 * t) = hi;
    }
    if (t == 0)
        scales[row * nb + b] = d;
}

// The rotation of one block (span ROT = 0: none, 32, 64, 128): lane t holds
// elements {4t..4t+3} and {16+4t..16+4t+3} (v[0..3], v[4..7]); h = 1, 2
// inside the lane, h = 4 with lane t^1, h = 8 with t^2 (the lane with the
// bit clear is lower), h = 16 inside the lane (v[i] with v[i+4]), h = 32, 64
// with the adjacent quads of a longer span; then times fp32(1/sqrt(ROT)).
template <int ROT>
__device__ __forceinline__ void rotate_p(float (&v)[8], int t, int lane)
{
    if constexpr (ROT != 0) {
#pragma unroll
        for (int base = 0; base < 8; base += 4) {
            const float a0 = v[base], a1 = v[base + 1], a2 = v[base + 2], a3 = v[base + 3];
            v[base] = a0 + a1;
            v[base + 1] = a0 - a1;
            v[base + 2] = a2 + a3;
            v[base + 3] = a2 - a3;
        }
#pragma unroll
        for (int base = 0; base < 8; base += 4) {
            const float a0 = v[base], a1 = v[base + 1], a2 = v[base + 2], a3 = v[base + 3];
            v[base] = a0 + a2;
            v[base + 2] = a0 - a2;
            v[base + 1] = a1 + a3;
            v[base + 3] = a1 - a3;
        }
        cross_stage<kQuadXor1>(v, (t & 1) != 0);
        cross_stage<kQuadXor2>(v, (t & 2) != 0);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float a = v[i], c = v[i + 4];
            v[i] = a + c;
            v[i + 4] = a - c;
        }
        if constexpr (ROT >= 64)
            cross_quad_stage<kSwzXor4>(v, (lane & 4) != 0);
        if constexpr (ROT >= 128)
            cross_quad_stage<kSwzXor8>(v, (lane & 8) != 0);
        const float c = ROT == 64 ? 0.125f
                                  : __uint_as_float(ROT == 128 ? 0x3DB504F3u : 0x3E3504F3u);
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = v[i] * c;
    }
}

// R rounds of 16 blocks per wave, one quad per block, in phases over the
// rounds (loads, rotations, block maxima, scales, codes, stores) so that the
// rounds' dependency chains overlap.  Block b of row `row` of round r is
// block 16 (R wave + r) + quad of the flattened matrix.  In the last wave,
// quads past the end repeat the last block's arithmetic and store nothing
// (a span never straddles the end, so every exchange between quads stays
// between quads of the same kind).
template <typename T, int BITS, int ROT, int R, typename I>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const T *__restrict__ x, int64_t k, int64_t ldx, int64_t nblk_total,
    uint8_t *__restrict__ codes, float *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int t = lane & 3, qd = lane >> 2;
    const I nb = (I)(k / 32);
    const I total = (I)nblk_total;
    const I wave = (I)blockIdx.x * (kThreads / 64) +
                   (I)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    I row[R], bk[R];
    bool live[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const I first = wave * (16 * R) + 16 * r; // uniform
        I blk = first + qd;
        live[r] = blk < total;
        blk = live[r] ? blk : total - 1;
        if (sizeof(I) == 4 && nb >= 16 && first + 15 < total) {
            // the division on the scalar unit: the quads' blocks are in the
            // first block's row or the next
            const I r0 = first / nb;
            const I b0 = first - r0 * nb;
            const I b = b0 + qd;
            row[r] = b < nb ? r0 : r0 + 1;
            bk[r] = b < nb ? b : b - nb;
        } else {
            row[r] = blk / nb;
            bk[r] = blk - row[r] * nb;
        }
    }
    float v[R][8];
#pragma unroll
    for (int r = 0; r < R; r++)
        load8(x + (int64_t)row[r] * ldx + (int64_t)bk[r] * 32, t, v[r]);
#pragma unroll
    for (int r = 0; r < R; r++)
        rotate_p<ROT>(v[r], t, lane);

    constexpr float kQmax = BITS == 4 ? 7.0f : 127.0f;
    constexpr float kQmin = BITS == 4 ? -8.0f : -127.0f;
    float d[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++)
            amax = fmaxf(amax, fabsf(v[r][i]));
        amax = fmaxf(amax, quad_swap<kQuadXor1>(amax));
        amax = fmaxf(amax, quad_swap<kQuadXor2>(amax));
        // IEEE division; an all-zero block has scale 0, and so has a block
        // whose amax / kQmax underflows (both get codes 0 below)
        d[r] = amax / kQmax;
    }
    // rint(v / d) with the IEEE quotient, taken first as v * rcp(d): its
    // error is below |v/d| * 3 * 2^-24 <= 2.3e-5 (|v/d| <= 127), so wherever
    // that product lies at least 1e-4 from a half-integer it rounds to the
    // same integer as the correctly rounded quotient.  The rare values within
    // that band, and scales too small for the reciprocal, make the whole wave
    // take the division (one uniform branch).
    float qv[R][8];
    bool slow = false;
#pragma unroll
    for (int r = 0; r < R; r++) {
        const float rd = __builtin_amdgcn_rcpf(d[r]);
        slow |= d[r] != 0.0f && !(d[r] >= 0x1p-100f);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            qv[r][i] = v[r][i] * rd;
            slow |= fabsf(fabsf(qv[r][i] - rintf(qv[r][i])) - 0.5f) < 1e-4f;
        }
    }
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int i = 0; i < 8; i++)
                qv[r][i] = v[r][i] / d[r];
    }
    uint2 out[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float c = d[r] != 0.0f ? rintf(qv[r][i]) : 0.0f;
            q[i] = (int)fminf(fmaxf(c, kQmin), kQmax);
        }
        if constexpr (BITS == 4) {
            // byte 4t+i = code(4t+i) low nibble | code(16+4t+i) high nibble
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; i++)
                word |= (uint32_t)((q[i] & 0xF) | ((q[i + 4] & 0xF) << 4)) << (8 * i);
            out[r].x = word;
            out[r].y = 0;
        } else {
            out[r].x = out[r].y = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                out[r].x |= (uint32_t)(q[i] & 0xFF) << (8 * i);
                out[r].y |= (uint32_t)(q[i + 4] & 0xFF) << (8 * i);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        if (!live[r])
            continue;
        if constexpr (BITS == 4) {
            *reinterpret_cast<uint32_t *>(codes + (int64_t)row[r] * (k / 2) + (int64_t)bk[r] * 16 +
                                          4 * t) = out[r].x;
        } else {
            uint8_t *dst = codes + (int64_t)row[r] * k + (int64_t)bk[r] * 32;
            *reinterpret_cast<uint32_t *>(dst + 4 * t) = out[r].x;
            *reinterpret_cast<uint32_t *>(dst + 16 + 4 * t) = out[r].y;
        }
        if (t == 0)
            scales[(int64_t)row[r] * nb + bk[r]] = d[r];
    }
}

template <typename T, int BITS, int ROT>
void launch_rows(dim3 grid, const T *x, int64_t k, int64_t ldx, int64_t nblk, uint8_t *codes,
                 float *scales, hipStream_t stream)
{
    constexpr int R = kQuantRounds;
    if (nblk + 16 * R * kThreads < ((int64_t)1 << 31))
        quantize_rows_kernel<T, BITS, ROT, R, uint32_t><<<grid, kThreads, 0, stream>>>(
            x, k, ldx, nblk, codes, scales);
    else
        quantize_rows_kernel<T, BITS, ROT, R, int64_t><<<grid, kThreads, 0, stream>>>(
            x, k, ldx, nblk, codes, scales);
}

template <typename T, int BITS>
void launch_rows_rot(dim3 grid, const T *x, int64_t k, int64_t ldx, int64_t nblk, int rot,
                     uint8_t *codes, float *scales, hipStream_t stream)
{
    switch (rot) {
    case 0: launch_rows<T, BITS, 0>(grid, x, k, ldx, nblk, codes, scales, stream); break;
    case 64: launch_rows<T, BITS, 64>(grid, x, k, ldx, nblk, codes, scales, stream); break;
    case 128: launch_rows<T, BITS, 128>(grid, x, k, ldx, nblk, codes, scales, stream); break;
    default: launch_rows<T, BITS, 32>(grid, x, k, ldx, nblk, codes, scales, stream); break;
    }
}

// ---- SwiGLU feeding the down projection of an expert layer.  The pages say
// only that the route covers the expert matmuls ("Where the engine is going:
// HRX and the NPU", section "4-bit activations reach the MoE experts"); the
// down projection's input h = silu(gate) * up is rotated and quantized like
// any activation, in the same kernel.

// e^x in fp32, every step one correctly rounded fp32 operation (the file is
// compiled without contraction): Cody-Waite range reduction n = rint(x log2 e),
// r = (x - n ln2_hi) - n ln2_lo (ln2_hi has 16 significant bits, so n ln2_hi
// is exact), the degree-6 Taylor polynomial of e^r in Horner form, then a
// scaling by 2^n.  x is clamped to [-87, 88].
__device__ __forceinline__ float exp_f32(float x)
{
    x = fminf(fmaxf(x, -87.0f), 88.0f);
    const float log2e = (float)1.4426950408889634;
    const float ln2_hi = 0.693145751953125f;
    const float ln2_lo = (float)(0.6931471805599453 - 0.693145751953125);
    const float n = rintf(x * log2e);
    const float r = (x - n * ln2_hi) - n * ln2_lo;
    float p = 1.0f / 720.0f;
    p = p * r + 1.0f / 120.0f;
    p = p * r + 1.0f / 24.0f;
    p = p * r + 1.0f / 6.0f;
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    return ldexpf(p, (int)n);
}

// silu(g) = g / (1 + e^-g), IEEE division
__device__ __forceinline__ float silu_f32(float g)
{
    const float den = 1.0f + exp_f32(-g);
    return g / den;
}

// One quad of lanes per 32-block of h, grid-stride; all four lanes of a quad
// walk the same blocks (the DPP exchanges stay inside the quad).
template <int BITS>
__global__ __launch_bounds__(kThreads) void swiglu_quantize_kernel(
    const float *__restrict__ gu, int64_t inter, int64_t ldgu, int64_t nblk_total,
    uint8_t *__restrict__ codes, float *__restrict__ scales)
{
    const int t = threadIdx.x & 3;
    const int64_t nb = inter / 32;
    const int64_t stride = (int64_t)gridDim.x * (kThreads / 4);
    for (int64_t blk = (int64_t)blockIdx.x * (kThreads / 4) + (threadIdx.x >> 2); blk < nblk_total;
         blk += stride) {
        const int64_t row = blk / nb, b = blk - row * nb;
        float g[8], u[8], v[8];
        load8(gu + row * ldgu + b * 32, t, g);
        load8(gu + row * ldgu + inter + b * 32, t, u);
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = silu_f32(g[i]) * u[i];
        quantize_block<BITS>(v, t, 32, row, b, inter, nb, codes, scales);
    }
}

} // namespace

hipError_t launch_swiglu_quantize(const float *gu, int64_t rows, int64_t inter, int64_t ldgu,
                                  int act_bits, void *codes, float *scales, hipStream_t stream)
{
    const int64_t nblk = rows * (inter / 32);
    if (nblk == 0)
        return hipSuccess;
    const int64_t needed = (nblk + kThreads / 4 - 1) / (kThreads / 4);
    const dim3 grid((unsigned)(needed < 2048 ? needed : 2048));
    uint8_t *c = static_cast<uint8_t *>(codes);
    if (act_bits == 4)
        swiglu_quantize_kernel<4><<<grid, kThreads, 0, stream>>>(gu, inter, ldgu, nblk, c, scales);
    else
        swiglu_quantize_kernel<8><<<grid, kThreads, 0, stream>>>(gu, inter, ldgu, nblk, c, scales);
    return hipGetLastError();
}

hipError_t launch_quantize(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx,
                           int act_bits, int rot, void *codes, float *scales,
                           hipStream_t stream)
{
    const int64_t nblk = m * (k / 32);
    if (nblk == 0)
        return hipSuccess;
    constexpr int R = kQuantRounds;
    const int64_t waves = (nblk + 16 * R - 1) / (16 * R);
    const int64_t wgs = (waves + kThreads / 64 - 1) / (kThreads / 64);
    if (wgs >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    uint8_t *c = static_cast<uint8_t *>(codes);
    if (dtype == 0 && act_bits == 4)
        launch_rows_rot<float, 4>(grid, static_cast<const float *>(x), k, ldx, nblk, rot, c, scales,
                                  stream);
    else if (dtype == 0)
        launch_rows_rot<float, 8>(grid, static_cast<const float *>(x), k, ldx, nblk, rot, c, scales,
                                  stream);
    else if (act_bits == 4)
        launch_rows_rot<uint16_t, 4>(grid, static_cast<const uint16_t *>(x), k, ldx, nblk, rot, c,
                                     scales, stream);
    else
        launch_rows_rot<uint16_t, 8>(grid, static_cast<const uint16_t *>(x), k, ldx, nblk, rot, c,
                                     scales, stream);
    return hipGetLastError();
}

} // namespace bpg
