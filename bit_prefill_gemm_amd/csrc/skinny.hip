// skinny.hip -- the W4A4 / W4A8 product for a few rows (M <= 32): a weight
// stream (gfx950).
//
// "509 tokens a second of prompt: the Hadamard route ships", section "Why
// prompts are a matrix-unit problem": with only a handful of rows every
// weight byte is used for a few multiply-adds, so the product is bound by how
// fast the Q4_0 weight image streams from HBM, not by the matrix unit.  This
// kernel is shaped for that:
//   - one workgroup per 32-column image tile; its NW waves split K into
//     contiguous ranges of groups of four blocks, so every wave streams its
//     own run of the tile (32 columns x 4 blocks x 18 bytes per group);
//   - every load is 16 (or 8) bytes wide: the weight image interleaves four
//     blocks, so one read per lane and 16-column tile holds that lane's
//     matrix operands for the group's four blocks; an activation read holds
//     one block of one row and a 4x4 transpose across the lane rows (gfx950
//     permlane swaps) turns four of them into the operands of four blocks;
//   - weight operands go straight from global memory into registers (no
//     barriers in the main loop), with D groups of loads in flight per wave
//     while a group is computed;
//   - the few activation rows are staged once per workgroup in LDS when they
//     and the transposed row scales fit 64 KB (16 rows, K <= 6528 with 4-bit
//     codes, K <= 3616 with 8-bit ones): read with whole cache lines and
//     stored with a padded row stride, so a wave's operand read of 16 rows
//     hits 16 distinct bank groups.  Read from L2 with every group instead,
//     each 16-lane quarter of an activation load touches 16 rows, i.e. 16
//     separate lines for 256 bytes, and those requests slow the weight stream
//     itself (16 x 5120 x 17408: 15.9 us per launch with the rows from L2,
//     14.9 us staged).  Larger K re-reads the rows from L2;
//   - the row scales are staged once per workgroup in LDS, transposed, so the
//     epilogue reads four rows' scales with one LDS read;
//   - the partial sums of the waves are added in a fixed order (wave 0, 1,
//     ...) through LDS, so the result is bit-identical from run to run.
// The per-block arithmetic is the one of the tiled kernel: operands widened
// to 16 x value, one v_mfma_i32_16x16x32_i8 per 16x16 tile and block with the
// accumulator input 0x4B400000, then t = fma(F, dw, -12582912*dw) (exact) and
// acc = fma(t, da, acc).  Rows past M repeat the last row; their sums reach
// only outputs that are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "operands.h"

namespace bpg {

namespace {

template <int BITS_, int TM_, int NW_, int TN_, int D_, bool AL_>
struct SkCfg {
    static constexpr int BITS = BITS_, TM = TM_, NW = NW_;
    static constexpr int TN = TN_;                    // 16-column tiles per workgroup: one image tile
    static_assert(TN == 2, "one 32-column image tile per workgroup");
    static constexpr int kCols = 16 * TN;
    // groups of four blocks in flight per wave: one when a wave walks many
    // groups and reads its activation rows from L2, two otherwise.  Deeper
    // rings measured slower, even for the weight stream alone: with every
    // wave of the grid streaming, more outstanding reads only lengthen the
    // memory queues (the waves of a SIMD still overlap one another's waits).
    static constexpr int D = D_;
    static constexpr int kThreads = 64 * NW;
    static constexpr int kRows = 16 * TM;             // rows covered (M <= kRows)
    static constexpr int kAB = BITS == 4 ? 16 : 32;   // code bytes per (row, block)
    static constexpr int kAH = kAB / 16;              // 16-byte halves per (row, block)
    static constexpr int kShift = BITS == 4 ? 8 : 4;  // log2 of the operand widening
    static constexpr int kR = TM * TN * 4;            // accumulators per lane
    static constexpr int kLdsRed = NW * kR * 64 * 4;  // bytes for the final reduction
    // activation rows staged once per workgroup in LDS (row stride padded by
    // 16 bytes, so that the 16 rows of an operand read fall in distinct banks)
    // instead of being re-read from L2 with every group
    static constexpr bool AL = AL_;
};

// The same address in every lane, made visibly uniform (scalar registers).
typedef const __attribute__((address_space(1))) uint8_t *gptr;

__device__ __forceinline__ gptr uniform_ptr(const void *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return (gptr)(((uint64_t)hi << 32) | lo);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 gload16(gptr base, uint32_t off)
{
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)(base + off);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 4x4 transpose across the four 16-lane rows of a wave: on entry register q
// of row g holds element (g, q); on exit it holds element (q, g).  Two
// 32-lane swaps exchange the off-diagonal 2x2 quadrants, two 16-lane swaps
// the off-diagonal elements inside each quadrant.
__device__ __forceinline__ void transpose_rows4(uint4 &v)
{
    auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    v = make_uint4(c[0], c[1], d[0], d[1]);
}

template <class C>
__global__ __launch_bounds__(C::kThreads) void skinny_kernel(GemmProblem p)
{
    constexpr int TM = C::TM, TN = C::TN, D = C::D, NW = C::NW, NT = C::kThreads;
    constexpr int kRows = C::kRows, kAB = C::kAB, kAH = C::kAH, R = C::kR;
    extern __shared__ __attribute__((aligned(16))) float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 15; // operand row / column inside a 16x16 tile
    const int g = lane >> 4; // operand K group (dword g of a block); result row group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int B = (int)(p.k / 32); // the host limits K
    const int NG = (B + 3) / 4;    // groups of four blocks
    const int rows = (int)p.rows;  // 1 .. kRows
    const int64_t tile = blockIdx.x;
    const int64_t col0 = tile * C::kCols;

    float *Da = lds;
    // staged activation rows (AL): row m at act_lds + m * a_stride bytes
    const int a_stride = (int)(p.k * kAB / 32) + 16;
    uint8_t *act_lds = reinterpret_cast<uint8_t *>(lds) + (size_t)4 * NG * kRows * 4;

    // ---- this wave's groups and its operand offsets.  Per group and lane:
    //      weights: one 16-byte read per 16-column tile = slot g of column c
    //      for the group's four blocks (the image interleaves them so);
    //      scales: 8 bytes = the four blocks' scales of column c;
    //      activations: 16 bytes = block 4G+g of row c, turned by a 4x4
    //      transpose across the lane rows into slot g of the four blocks.
    const int g0 = (int)((int64_t)wave * NG / NW);
    const int g1 = (int)((int64_t)(wave + 1) * NG / NW);
    const int64_t arow = p.k * kAB / 32;
    const gptr a_base = uniform_ptr(p.codes);
    const gptr w_base = uniform_ptr(p.wcodes + (col0 / 32) * NG * 2304);
    uint32_t va[TM], vw[TN];
    // the group's scales: 16 bytes at [c16 = c] = column c's and column
    // 16 + c's four blocks
    const uint32_t vdw = (uint32_t)(2048 + c * 16);
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int m = 16 * i + c;
        va[i] = (uint32_t)((m < rows ? m : rows - 1) * arow);
    }
#pragma unroll
    for (int j = 0; j < TN; j++) {
        // 16-column tile j is half j of the image tile
        vw[j] = (uint32_t)((g * 32 + 16 * j + c) * 16);
    }

    // ring of D groups of operands in registers
    uint4 rw[D][TN], ra[C::AL ? 1 : D][TM][kAH], rdw[D];
    auto load = [&](int d, int G) {
        const gptr wb = w_base + G * 2304;
        // the last group may end past block B-1: those lanes re-read block B-1
        const int bq = min(4 * G + g, B - 1);
#pragma unroll
        for (int j = 0; j < TN; j++)
            rw[d][j] = gload16(wb, vw[j]);
        rdw[d] = gload16(wb, vdw);
        if constexpr (!C::AL) {
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int h = 0; h < kAH; h++)
                    ra[d][i][h] = gload16(a_base, va[i] + bq * kAB + 16 * h);
        }
    };

    float acc[TM][TN][4];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                acc[i][j][r] = 0.0f;
    v4i magic;
#pragma unroll
    for (int r = 0; r < 4; r++)
        magic[r] = kMagicBits;

    // One group: the matrix products of its four blocks first, then their
    // epilogues, so that no result is read right after its instruction.  The
    // last group may hold blocks past B: the image gives them scale 0 and LDS
    // row scale 0, so they add exactly zero.
    auto compute = [&](int d, int G) {
        const int ad = C::AL ? 0 : d; // the activation operands' slot
        if constexpr (C::AL) {
            // from the staged rows: block 4G+g of row c (blocks past B re-read B-1)
            const int bq = min(4 * G + g, B - 1);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int h = 0; h < kAH; h++)
                    ra[0][i][h] = *reinterpret_cast<const uint4 *>(act_lds + (16 * i + c) * a_stride +
                                                                   bq * kAB + 16 * h);
        }
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int h = 0; h < kAH; h++)
                transpose_rows4(ra[ad][i][h]);
        v4i s[4][TN][TM];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            long a[TM];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const uint32_t lo = q == 0 ? ra[ad][i][0].x : q == 1 ? ra[ad][i][0].y
                                  : q == 2 ? ra[ad][i][0].z : ra[ad][i][0].w;
                const uint32_t hi = q == 0 ? ra[ad][i][kAH - 1].x : q == 1 ? ra[ad][i][kAH - 1].y
                                  : q == 2 ? ra[ad][i][kAH - 1].z : ra[ad][i][kAH - 1].w;
                // 4-bit: low and high nibbles of dword g; 8-bit: bytes 4g.. and 16+4g..
                a[i] = kAH == 1 ? pack2(act_lo(lo), act_hi(lo)) : pack2(lo, hi);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const uint32_t wd = q == 0 ? rw[d][j].x : q == 1 ? rw[d][j].y
                                  : q == 2 ? rw[d][j].z : rw[d][j].w;
                const long w = pack2(q40_lo(wd), q40_hi(wd));
#pragma unroll
                for (int i = 0; i < TM; i++)
                    s[q][j][i] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[i], w, magic, 0, 0, 0);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int b = 4 * G + q;
            float4 da[TM];
#pragma unroll
            for (int i = 0; i < TM; i++)
                da[i] = *reinterpret_cast<const float4 *>(Da + b * kRows + 16 * i + 4 * g);
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const uint32_t hp = j == 0 ? (q < 2 ? rdw[d].x : rdw[d].y) : (q < 2 ? rdw[d].z : rdw[d].w);
                const uint16_t hb = (uint16_t)((q & 1) ? hp >> 16 : hp & 0xFFFFu);
                const float dw = half_bits_to_float(hb);
                const float cm = -kMagic * dw; // exact: dw has 11 significant bits
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    const float dq[4] = {da[i].x, da[i].y, da[i].z, da[i].w};
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const float t = __builtin_fmaf(__int_as_float(s[q][j][i][r]), dw, cm);
                        acc[i][j][r] = __builtin_fmaf(t, dq[r], acc[i][j][r]);
                    }
                }
            }
        }
    };

    // Every slot is refilled right after its group is computed, so D groups
    // of loads are always in flight.  The loads are unconditional (groups past
    // the wave's range re-read its last group and are never computed), which
    // keeps the order of outstanding loads the same in every iteration; the
    // scheduling barriers keep the prologue's loads in that same slot order.
    // Activation scales, transposed to [block][row]; zero past M and for the
    // blocks of the last group past B.  A thread takes block columns b = tid,
    // tid + NT, ... and all kRows rows of each (coalesced reads along b, no
    // index division).  The first column's loads are issued before the
    // operand prologue and stored behind it, so both latencies overlap.
    const int da_cols = 4 * NG;
    float dv[kRows];
    auto da_load = [&](int b) {
#pragma unroll
        for (int m = 0; m < kRows; m++)
            dv[m] = b < B && m < rows ? p.scales[(int64_t)m * B + b] : 0.0f;
    };
    auto da_store = [&](int b) {
        if (b < da_cols)
#pragma unroll
            for (int m = 0; m < kRows; m++)
                Da[b * kRows + m] = dv[m];
    };
    // activation rows (AL): thread t copies 16-byte chunks t, t + NT, ... of
    // every row (rows past M repeat the last row), full cache lines per wave
    const int cpr = (int)(p.k * kAB / 32 / 16); // 16-byte chunks per row
    uint4 av[C::AL ? kRows : 1];
    auto act_load = [&](int ch) {
        if (ch < cpr)
#pragma unroll
            for (int m = 0; m < kRows; m++)
                av[m] = gload16(a_base, (uint32_t)((m < rows ? m : rows - 1) * arow) + (uint32_t)ch * 16u);
    };
    auto act_store = [&](int ch) {
        if (ch < cpr)
#pragma unroll
            for (int m = 0; m < kRows; m++)
                *reinterpret_cast<uint4 *>(act_lds + m * a_stride + ch * 16) = av[m];
    };
    da_load(tid);
    if constexpr (C::AL)
        act_load(tid);
    __builtin_amdgcn_sched_barrier(0);

    // The wave walks its groups starting at an offset that depends on the
    // tile, so that the workgroups of different tiles, which all read the
    // same few activation rows, do not read the same lines at the same time.
    const int ng = g1 - g0;
    const int rot = ng > 0 ? (int)(tile % ng) : 0;
    auto group_at = [&](int k) { // k-th group of the walk; clamped to the last one
        if (ng <= 0)
            return min(g0, NG - 1);
        const int r = min(k, ng - 1) + rot;
        return g0 + (r >= ng ? r - ng : r);
    };
#pragma unroll
    for (int d = 0; d < D; d++) {
        load(d, group_at(d));
        __builtin_amdgcn_sched_barrier(0);
    }

    da_store(tid);
    for (int b = tid + NT; b < da_cols; b += NT) {
        da_load(b);
        da_store(b);
    }
    if constexpr (C::AL) {
        act_store(tid);
        for (int ch = tid + NT; ch < cpr; ch += NT) {
            act_load(ch);
            act_store(ch);
        }
    }
    __syncthreads(); // the scales (and the staged rows) in LDS

    for (int base = 0; base < ng; base += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            const int k = base + d;
            if (k < ng)
                compute(d, group_at(k));
            load(d, group_at(k + D));
        }
    }

    // ---- fixed-order sum over the waves (wave 0, 1, ...); widening removed
    __syncthreads(); // every wave is done with the scales
    float *red = lds;
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                red[(wave * R + (i * TN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    __syncthreads();
    const float unscale = 1.0f / (float)(1 << C::kShift);
    for (int v = tid; v < R * 64; v += NT) {
        float s = red[v];
#pragma unroll
        for (int w = 1; w < NW; w++)
            s += red[w * R * 64 + v];
        const int q = v >> 6, ln = v & 63;
        const int i = q / (TN * 4), j = (q / 4) % TN, r = q % 4;
        const int m = 16 * i + 4 * (ln >> 4) + r;
        if (m < rows)
            store_y(p, (int64_t)m * p.ldy + col0 + 16 * j + (ln & 15), s * unscale);
    }
}

template <class C>
size_t skinny_lds(const GemmProblem &p)
{
    size_t bytes = (size_t)((p.k / 32 + 3) / 4) * 4 * C::kRows * 4;
    if (C::AL)
        bytes += (size_t)C::kRows * (size_t)(p.k * C::kAB / 32 + 16);
    return bytes > (size_t)C::kLdsRed ? bytes : (size_t)C::kLdsRed;
}

template <class C>
hipError_t launch_cfg(const GemmProblem &p, hipStream_t stream)
{
    const size_t lds = skinny_lds<C>(p);
    skinny_kernel<C><<<dim3((unsigned)(p.n / C::kCols)), C::kThreads, lds, stream>>>(p);
    return hipGetLastError();
}

template <int BITS, int TM, int TN, int D, bool AL>
hipError_t launch_nw(const GemmProblem &p, int nw, hipStream_t stream)
{
    if (nw == 4)
        return launch_cfg<SkCfg<BITS, TM, 4, TN, D, AL>>(p, stream);
    if constexpr (TM == 1) {
        if (nw == 16)
            return launch_cfg<SkCfg<BITS, TM, 16, TN, D, AL>>(p, stream);
    }
    return launch_cfg<SkCfg<BITS, TM, 8, TN, D, AL>>(p, stream);
}

// Activation rows staged in LDS: one row tile whose rows and transposed
// scales fit the 64 KB of dynamic LDS.
template <int TM>
bool stage_rows(const GemmProblem &p)
{
    if (TM != 1)
        return false;
    const int64_t da = (p.k / 32 + 3) / 4 * 4 * 16 * 4;
    const int64_t rows = 16 * (p.k * (p.act_bits == 4 ? 16 : 32) / 32 + 16);
    return da + rows <= 65536;
}

template <int BITS, int TM, int TN, int D>
hipError_t launch_al(const GemmProblem &p, int nw, hipStream_t stream)
{
    if constexpr (TM == 1) {
        if (stage_rows<TM>(p))
            return launch_nw<BITS, TM, TN, D, true>(p, nw, stream);
    }
    return launch_nw<BITS, TM, TN, D, false>(p, nw, stream);
}

// Waves per workgroup: enough waves in the whole grid to keep the weight
// stream busy (about 8 per CU), each with at least 4 groups of K.
template <int BITS, int TM, int TN>
hipError_t launch_tn(const GemmProblem &p, hipStream_t stream)
{
    const int64_t tiles = p.n / (16 * TN), NG = (p.k / 32 + 3) / 4;
    // (two row tiles need more registers: at most 8 waves)
    constexpr int nw_max = TM == 1 ? 16 : 8;
    int nw = 4;
    while (nw < nw_max && tiles * nw < 2048 && NG / (2 * nw) >= 4)
        nw *= 2;
    // two groups in flight with staged rows (the operand loads are the weights
    // alone) or with few groups per wave; one otherwise
    if (NG / nw <= 6 || stage_rows<TM>(p))
        return launch_al<BITS, TM, TN, 2>(p, nw, stream);
    return launch_nw<BITS, TM, TN, 1, false>(p, nw, stream);
}

template <int BITS, int TM>
hipError_t launch_tm(const GemmProblem &p, hipStream_t stream)
{
    return launch_tn<BITS, TM, 2>(p, stream);
}

} // namespace

bool skinny_fits(const GemmProblem &p)
{
    if (p.rows < 1 || p.rows > 32)
        return false;
    const int rows_cov = p.rows <= 16 ? 16 : 32;
    // the transposed scales (whole groups of four blocks) must fit the 64 KB
    // of dynamic LDS
    return (p.k / 32 + 3) / 4 * 4 * rows_cov * 4 <= 65536;
}

hipError_t launch_skinny(const GemmProblem &p, hipStream_t stream)
{
    if (p.act_bits == 4)
        return p.rows <= 16 ? launch_tm<4, 1>(p, stream) : launch_tm<4, 2>(p, stream);
    return p.rows <= 16 ? launch_tm<8, 1>(p, stream) : launch_tm<8, 2>(p, stream);
}

} // namespace bpg
