// gemm.hip -- W4A4 / W4A8 products on CDNA4 integer matrix cores (gfx950).
//
// "509 tokens a second of prompt: the Hadamard route ships", section "Why
// prompts are a matrix-unit problem": prompts are a matrix-unit workload; a
// Q4_0 code u means u-8, which is the code with its top bit flipped read as a
// 4-bit two's-complement number, so the kernel reads Q4_0 nibbles bit for bit.
// gfx950 has no int4 matrix instruction, so both operands are widened to int8
// in registers and each 32-value block is one v_mfma_i32_32x32x32_i8 per
// 32x32 output tile.
//
// Per K-block b the kernel needs y[m][n] += da[m][b] * dw[n][b] * S[m][n][b]
// with S the exact int32 block dot product:
//   - operands are widened as 16*value (a nibble in the top half of a byte),
//     so the instruction returns 256*S (8-bit activations: 16*S); the power
//     of two is folded into the weight scale;
//   - the accumulator input is 0x4B400000 (1.5*2^23 as fp32), so the int32
//     result, read as fp32, is exactly 12582912 + 256*S (|256*S| < 2^22);
//   - t = fma(F, dws, -12582912*dws) = 256*S*dws (the constant product is exact
//     because dws carries at most 11 significant bits), then
//     acc = fma(t, da, acc).
// That is two fp32 VALU operations per (m, n, b) and no integer conversion.
// The block sums themselves are exposed through the same main loop
// (MODE kSums) for bit-exact parity checks.
//
// Data flow: activation codes [rows][k/2] (or [rows][k]) and the weight image
// ([N/32][B][32][16 B] nibbles + fp16 scales) are staged through LDS, KC
// blocks per stage, double buffered, laid out so that every wave reads its
// MFMA operands as one contiguous 512-byte run per instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bpg {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

enum Mode { kGemm = 0, kGrouped = 1, kSums = 2 };

template <int BITS_, int BM_, int BN_, int KC_, int WM_, int WN_, int WK_>
struct Cfg {
    static constexpr int BITS = BITS_, BM = BM_, BN = BN_, KC = KC_;
    static constexpr int WM = WM_, WN = WN_, WK = WK_;
    static constexpr int kWaves = WM * WN * WK;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int TM = BM / (32 * WM);
    static constexpr int TN = BN / (32 * WN);
    static constexpr int kAB = BITS == 4 ? 16 : 32;  // activation code bytes per (row, block)
    static constexpr int kShift = BITS == 4 ? 8 : 4; // log2 of the operand widening factor
    static constexpr int kLdsA = KC * BM * kAB;
    static constexpr int kLdsW = KC * BN * 16;
    static constexpr int kLdsAs = KC * BM * 4;
    static constexpr int kLdsWs = KC * BN * 8;
    static constexpr int kLdsBuf = kLdsA + kLdsW + kLdsAs + kLdsWs;
    static constexpr int kLdsRed = WM * WN * (WK - 1) * 1024 * 4;
    static constexpr int kLds = (2 * kLdsBuf > kLdsRed ? 2 * kLdsBuf : kLdsRed);
    static constexpr int kChunksA = BM * KC * (kAB / 16); // 16-byte chunks per stage
    static constexpr int kChunksW = BN * KC;
    static constexpr int kPerThreadA = (kChunksA + kThreads - 1) / kThreads;
    static constexpr int kPerThreadW = (kChunksW + kThreads - 1) / kThreads;
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tiling");
    static_assert(KC % WK == 0, "K split");
    static_assert(kLds <= 65536, "LDS budget");
};

// Activation nibbles (already two's complement) -> 16*value in each byte.
__device__ __forceinline__ v4i widen_act4(uint2 r)
{
    v4i o;
    o[0] = (int)((r.x << 4) & 0xF0F0F0F0u);
    o[1] = (int)((r.y << 4) & 0xF0F0F0F0u);
    o[2] = (int)(r.x & 0xF0F0F0F0u);
    o[3] = (int)(r.y & 0xF0F0F0F0u);
    return o;
}

// Q4_0 nibbles u -> top bit flipped (u XOR 8 = u-8 in two's complement) -> 16*(u-8).
__device__ __forceinline__ v4i widen_q4_0(uint2 r)
{
    r.x ^= 0x88888888u;
    r.y ^= 0x88888888u;
    return widen_act4(r);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// Workgroups are dispatched round-robin over the 8 XCDs (w % 8 selects the
// XCD).  Hand each XCD a contiguous range of logical tiles so that the tiles
// sharing weight columns share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total)
{
    if (total % 8 != 0)
        return w;
    return (w % 8) * (total / 8) + w / 8;
}

// Grouped tiling: expert e owns ceil(rows_e / BM) consecutive row slots.  Find
// the expert and the row range of `slot` with a workgroup-wide scan over the
// clamped offsets.  Returns false (uniformly) if the slot lies beyond the last
// tile.  Every row range returned lies inside [0, rows).
template <int NT>
__device__ bool grouped_slot(const int32_t *__restrict__ off, int64_t experts, int64_t rows,
                             int bm, int slot, int *scan, int64_t &row0, int64_t &row_end,
                             int64_t &expert)
{
    __shared__ int64_t found[4];
    const int tid = threadIdx.x;
    if (tid == 0)
        found[0] = -1;
    int64_t carry = 0;
    for (int64_t base = 0; base < experts; base += NT) {
        const int64_t e = base + tid;
        int cnt = 0;
        int64_t a = 0, b = 0;
        if (e < experts) {
            a = off[e];
            b = off[e + 1];
            a = a < 0 ? 0 : (a > rows ? rows : a);
            b = b < 0 ? 0 : (b > rows ? rows : b);
            if (b > a)
                cnt = (int)((b - a + bm - 1) / bm);
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < NT; d <<= 1) { // inclusive Hillis-Steele scan
            const int v = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        const int64_t incl = carry + scan[tid];
        const int64_t excl = incl - cnt;
        if (cnt > 0 && slot >= excl && slot < incl) {
            found[0] = 1;
            found[1] = a + (slot - excl) * bm;
            found[2] = b;
            found[3] = e;
        }
        carry += scan[NT - 1];
        __syncthreads();
    }
    if (found[0] < 0)
        return false;
    row0 = found[1];
    row_end = found[2];
    expert = found[3];
    return true;
}

template <class C, int MODE>
__global__ __launch_bounds__(C::kThreads) void w4a4_kernel(GemmProblem p, int tiles_m,
                                                           int tiles_n, int tm0, int tn0)
{
    constexpr int BM = C::BM, BN = C::BN, KC = C::KC, TM = C::TM, TN = C::TN;
    constexpr int WN = C::WN, WK = C::WK, NT = C::kThreads, kAB = C::kAB;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rr = lane & 31;
    const int g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave % WK;
    const int wn = (wave / WK) % WN;
    const int wm = wave / (WK * WN);

    const int64_t B = p.k / 32;
    const int64_t ntiles32 = p.n / 32;

    // ---- which tile this workgroup computes
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    int64_t row0, row_end, col0, expert;
    if (MODE == kGrouped) {
        const int slot = L / tiles_n;
        col0 = (int64_t)(L % tiles_n) * BN;
        if (!grouped_slot<NT>(p.offsets, p.experts, p.rows, BM, slot,
                              reinterpret_cast<int *>(lds), row0, row_end, expert))
            return; // uniform across the workgroup
        __syncthreads(); // the scan area is reused by the stage buffers below
    } else {
        row0 = (int64_t)(tm0 + L % tiles_m) * BM;
        col0 = (int64_t)(tn0 + L / tiles_m) * BN;
        row_end = p.rows;
        expert = MODE == kSums ? p.expert : 0;
    }

    const uint8_t *__restrict__ wc = p.wcodes + expert * ntiles32 * B * 512;
    const uint16_t *__restrict__ ws = p.wscales + expert * ntiles32 * B * 32;
    const int64_t ct0 = col0 / 32;
    const int64_t arow_bytes = p.k * kAB / 32;

    // ---- staging registers
    uint4 ra[C::kPerThreadA];
    uint4 rw[C::kPerThreadW];
    constexpr int kPerThreadAs = (BM * KC + NT - 1) / NT;
    constexpr int kPerThreadWs = (BN * KC + NT - 1) / NT;
    float ras[kPerThreadAs];
    uint16_t rws[kPerThreadWs];

    auto load_stage = [&](int64_t kb0) {
#pragma unroll
        for (int i = 0; i < C::kPerThreadA; i++) {
            const int c = tid + i * NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < C::kChunksA) {
                const int row = c / (KC * (kAB / 16));
                const int rem = c % (KC * (kAB / 16));
                const int kc = rem / (kAB / 16), part = rem % (kAB / 16);
                const int64_t grow = row0 + row;
                if (grow < row_end && kb0 + kc < B)
                    v = *reinterpret_cast<const uint4 *>(p.codes + grow * arow_bytes +
                                                         (kb0 + kc) * kAB + part * 16);
            }
            ra[i] = v;
        }
#pragma unroll
        for (int i = 0; i < C::kPerThreadW; i++) {
            const int c = tid + i * NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < C::kChunksW) {
                const int ct = c / (KC * 32);
                const int rem = c % (KC * 32);
                const int kc = rem / 32, j = rem % 32;
                if (kb0 + kc < B)
                    v = *reinterpret_cast<const uint4 *>(
                        wc + (((ct0 + ct) * B + kb0 + kc) * 32 + j) * 16);
            }
            rw[i] = v;
        }
#pragma unroll
        for (int i = 0; i < kPerThreadAs; i++) {
            const int c = tid + i * NT;
            float v = 0.0f;
            if (c < BM * KC) {
                const int row = c / KC, kc = c % KC;
                const int64_t grow = row0 + row;
                if (MODE != kSums && grow < row_end && kb0 + kc < B)
                    v = p.scales[grow * B + kb0 + kc]; // block sums never read scales
            }
            ras[i] = v;
        }
#pragma unroll
        for (int i = 0; i < kPerThreadWs; i++) {
            const int c = tid + i * NT;
            uint16_t v = 0;
            if (c < BN * KC) {
                const int ct = c / (KC * 32);
                const int rem = c % (KC * 32);
                const int kc = rem / 32, j = rem % 32;
                if (kb0 + kc < B)
                    v = ws[((ct0 + ct) * B + kb0 + kc) * 32 + j];
            }
            rws[i] = v;
        }
    };

    auto store_stage = [&](int buf) {
        uint8_t *A = lds + buf * C::kLdsBuf;
        uint8_t *W = A + C::kLdsA;
        float *As = reinterpret_cast<float *>(W + C::kLdsW);
        float2 *Ws = reinterpret_cast<float2 *>(W + C::kLdsW + C::kLdsAs);
#pragma unroll
        for (int i = 0; i < C::kPerThreadA; i++) {
            const int c = tid + i * NT;
            if (c < C::kChunksA) {
                const int row = c / (KC * (kAB / 16));
                const int rem = c % (KC * (kAB / 16));
                const int kc = rem / (kAB / 16), part = rem % (kAB / 16);
                const int rt = row / 32, r = row % 32;
                const int base = (kc * (BM / 32) + rt) * (kAB / 8) + part * 2;
                *reinterpret_cast<uint2 *>(A + base * 256 + r * 8) = make_uint2(ra[i].x, ra[i].y);
                *reinterpret_cast<uint2 *>(A + (base + 1) * 256 + r * 8) =
                    make_uint2(ra[i].z, ra[i].w);
            }
        }
#pragma unroll
        for (int i = 0; i < C::kPerThreadW; i++) {
            const int c = tid + i * NT;
            if (c < C::kChunksW) {
                const int ct = c / (KC * 32);
                const int rem = c % (KC * 32);
                const int kc = rem / 32, j = rem % 32;
                const int base = (kc * (BN / 32) + ct) * 2;
                *reinterpret_cast<uint2 *>(W + base * 256 + j * 8) = make_uint2(rw[i].x, rw[i].y);
                *reinterpret_cast<uint2 *>(W + (base + 1) * 256 + j * 8) =
                    make_uint2(rw[i].z, rw[i].w);
            }
        }
#pragma unroll
        for (int i = 0; i < kPerThreadAs; i++) {
            const int c = tid + i * NT;
            if (c < BM * KC) {
                const int row = c / KC, kc = c % KC;
                As[kc * BM + row] = ras[i];
            }
        }
#pragma unroll
        for (int i = 0; i < kPerThreadWs; i++) {
            const int c = tid + i * NT;
            if (c < BN * KC) {
                const int ct = c / (KC * 32);
                const int rem = c % (KC * 32);
                const int kc = rem / 32, j = rem % 32;
                const float dws = half_bits_to_float(rws[i]) * (1.0f / (1 << C::kShift));
                Ws[kc * BN + ct * 32 + j] = make_float2(dws, -kMagic * dws);
            }
        }
    };

    // rows of each of this wave's 32-row tiles that hold data (wave-uniform)
    int vrows[TM];
#pragma unroll
    for (int i = 0; i < TM; i++) {
        int64_t v = row_end - (row0 + (int64_t)(wm * TM + i) * 32);
        vrows[i] = v < 0 ? 0 : (v > 32 ? 32 : (int)v);
    }

    float acc[TM][TN][16];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][j][r] = 0.0f;

    v16i magic;
#pragma unroll
    for (int r = 0; r < 16; r++)
        magic[r] = kMagicBits;

    const int64_t nstages = (B + KC - 1) / KC;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int64_t s = 0; s < nstages; s++) {
        const int buf = (int)(s & 1);
        const int64_t kb0 = s * KC;
        if (s + 1 < nstages)
            load_stage(kb0 + KC);

        const uint8_t *A = lds + buf * C::kLdsBuf;
        const uint8_t *W = A + C::kLdsA;
        const float *As = reinterpret_cast<const float *>(W + C::kLdsW);
        const float2 *Ws = reinterpret_cast<const float2 *>(W + C::kLdsW + C::kLdsAs);
        const int64_t kvalid = B - kb0; // blocks of this stage inside K (>= 1)

#pragma unroll
        for (int kk = 0; kk < KC / WK; kk++) {
            const int kc = kk * WK + wk;
            if (kc >= kvalid)
                break;
            v4i a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int base = (kc * (BM / 32) + wm * TM + i) * (kAB / 8);
                if (C::BITS == 4) {
                    a[i] = widen_act4(*reinterpret_cast<const uint2 *>(A + (base + g) * 256 + rr * 8));
                } else {
                    uint2 lo = *reinterpret_cast<const uint2 *>(A + (base + g) * 256 + rr * 8);
                    uint2 hi = *reinterpret_cast<const uint2 *>(A + (base + 2 + g) * 256 + rr * 8);
                    a[i][0] = (int)lo.x; a[i][1] = (int)lo.y;
                    a[i][2] = (int)hi.x; a[i][3] = (int)hi.y;
                }
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int base = (kc * (BN / 32) + wn * TN + j) * 2;
                b[j] = widen_q4_0(*reinterpret_cast<const uint2 *>(W + (base + g) * 256 + rr * 8));
            }

            v16i D[TM][TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    if (vrows[i] > 0)
                        D[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], magic, 0, 0, 0);

            if (MODE == kSums) {
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++) {
                        if (vrows[i] <= 0)
                            continue;
                        const int64_t col = col0 + (wn * TN + j) * 32 + rr;
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            const int64_t row = row0 + (wm * TM + i) * 32 + 8 * (r / 4) + 4 * g + (r % 4);
                            if (row >= p.m0 && row < p.m1 && col >= p.n0 && col < p.n1) {
                                const int32_t sv = (D[i][j][r] - kMagicBits) >> C::kShift;
                                p.sums[((row - p.m0) * (p.n1 - p.n0) + (col - p.n0)) * B + kb0 + kc] = sv;
                            }
                        }
                    }
            } else {
                float2 wsc[TN];
#pragma unroll
                for (int j = 0; j < TN; j++)
                    wsc[j] = Ws[kc * BN + (wn * TN + j) * 32 + rr];
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    if (vrows[i] <= 0)
                        continue;
                    float4 da[4];
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        da[q] = *reinterpret_cast<const float4 *>(
                            As + kc * BM + (wm * TM + i) * 32 + 8 * q + 4 * g);
#pragma unroll
                    for (int j = 0; j < TN; j++) {
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            if (8 * q >= vrows[i])
                                continue;
                            const float dq[4] = {da[q].x, da[q].y, da[q].z, da[q].w};
#pragma unroll
                            for (int e = 0; e < 4; e++) {
                                const int r = 4 * q + e;
                                const float t = __builtin_fmaf(__int_as_float(D[i][j][r]), wsc[j].x, wsc[j].y);
                                acc[i][j][r] = __builtin_fmaf(t, dq[e], acc[i][j][r]);
                            }
                        }
                    }
                }
            }
        }

        if (s + 1 < nstages)
            store_stage(buf ^ 1);
        __syncthreads();
    }

    if (MODE == kSums)
        return;

    // ---- deterministic reduction of the K split: wave wk=0 adds wk=1,2,... in order
    if (WK > 1) {
        float *red = reinterpret_cast<float *>(lds);
        const int grp = wm * WN + wn;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) {
                if (wk > 0) {
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        red[((grp * (WK - 1) + wk - 1) * 16 + r) * 64 + lane] = acc[i][j][r];
                }
                __syncthreads();
                if (wk == 0) {
                    for (int w = 1; w < WK; w++)
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            acc[i][j][r] += red[((grp * (WK - 1) + w - 1) * 16 + r) * 64 + lane];
                }
                __syncthreads();
            }
        if (wk > 0)
            return;
    }

#pragma unroll
    for (int i = 0; i < TM; i++) {
        if (vrows[i] <= 0)
            continue;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t col = col0 + (wn * TN + j) * 32 + rr;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int rl = 8 * (r / 4) + 4 * g + (r % 4);
                if (rl < vrows[i]) {
                    const int64_t row = row0 + (wm * TM + i) * 32 + rl;
                    p.y[row * p.ldy + col] = acc[i][j][r];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launchers

template <class C, int MODE>
hipError_t launch_cfg(const GemmProblem &p, int tiles_m, int tiles_n, int tm0, int tn0,
                      int64_t grid, hipStream_t stream)
{
    if (grid <= 0)
        return hipSuccess;
    w4a4_kernel<C, MODE><<<dim3((unsigned)grid), C::kThreads, 0, stream>>>(p, tiles_m, tiles_n,
                                                                            tm0, tn0);
    return hipGetLastError();
}

// Tile shapes.  Large M: 64x64 workgroup tiles, one 32x32 tile per wave.
// Small M (<= 32): one 32-row tile, 64 columns, K split over two waves.
template <int BITS> using CfgLarge = Cfg<BITS, 64, 64, 8, 2, 2, 1>;
template <int BITS> using CfgSmall = Cfg<BITS, 32, 64, 8, 1, 2, 2>;

template <int BITS>
hipError_t launch_dense_bits(const GemmProblem &p, hipStream_t stream)
{
    if (p.rows <= 32) {
        using C = CfgSmall<BITS>;
        const int tm = (int)((p.rows + C::BM - 1) / C::BM), tn = (int)(p.n / C::BN);
        if (p.n % C::BN == 0)
            return launch_cfg<C, kGemm>(p, tm, tn, 0, 0, (int64_t)tm * tn, stream);
    }
    using C = CfgLarge<BITS>;
    if (p.n % C::BN == 0) {
        const int tm = (int)((p.rows + C::BM - 1) / C::BM), tn = (int)(p.n / C::BN);
        return launch_cfg<C, kGemm>(p, tm, tn, 0, 0, (int64_t)tm * tn, stream);
    }
    using C32 = Cfg<BITS, 64, 32, 8, 2, 1, 1>; // N a multiple of 32 only
    const int tm = (int)((p.rows + C32::BM - 1) / C32::BM), tn = (int)(p.n / C32::BN);
    return launch_cfg<C32, kGemm>(p, tm, tn, 0, 0, (int64_t)tm * tn, stream);
}

template <int BITS>
hipError_t launch_grouped_bits(const GemmProblem &p, hipStream_t stream)
{
    using C = Cfg<BITS, 64, 32, 8, 2, 1, 1>;
    const int tn = (int)(p.n / C::BN);
    // every expert needs ceil(rows_e / BM) slots: bounded by both of these
    int64_t slots = (p.rows + p.experts * (C::BM - 1)) / C::BM;
    if (slots > p.rows)
        slots = p.rows;
    return launch_cfg<C, kGrouped>(p, 0, tn, 0, 0, slots * tn, stream);
}

template <int BITS>
hipError_t launch_sums_bits(const GemmProblem &p, hipStream_t stream)
{
    using C = Cfg<BITS, 64, 32, 8, 2, 1, 1>;
    const int tm0 = (int)(p.m0 / C::BM), tm1 = (int)((p.m1 + C::BM - 1) / C::BM);
    const int tn0 = (int)(p.n0 / C::BN), tn1 = (int)((p.n1 + C::BN - 1) / C::BN);
    const int tm = tm1 - tm0, tn = tn1 - tn0;
    return launch_cfg<C, kSums>(p, tm, tn, tm0, tn0, (int64_t)tm * tn, stream);
}

} // namespace

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream)
{
    if (p.rows == 0)
        return hipSuccess;
    return p.act_bits == 4 ? launch_dense_bits<4>(p, stream) : launch_dense_bits<8>(p, stream);
}

hipError_t launch_grouped_gemm(const GemmProblem &p, hipStream_t stream)
{
    if (p.rows == 0)
        return hipSuccess;
    return p.act_bits == 4 ? launch_grouped_bits<4>(p, stream) : launch_grouped_bits<8>(p, stream);
}

hipError_t launch_blocksums(const GemmProblem &p, hipStream_t stream)
{
    if (p.m1 <= p.m0 || p.n1 <= p.n0)
        return hipSuccess;
    return p.act_bits == 4 ? launch_sums_bits<4>(p, stream) : launch_sums_bits<8>(p, stream);
}

} // namespace bpg
