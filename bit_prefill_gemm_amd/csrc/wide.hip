// wide.hip -- the W4A4 product for many rows on 64 x 160 tiles (gfx950).
//
// "509 tokens a second of prompt: the Hadamard route ships", section "Why
// prompts are a matrix-unit problem": with hundreds of rows the product is
// matrix work.  On gfx950 the per-block scale epilogue (two fp32 VALU
// operations per output and block, see operands.h) is what bounds it, so this
// kernel is built to keep the VALU busy with that epilogue and little else:
//   - operands move from global memory to LDS with direct 16-byte (and, for
//     the row scales, 4-byte) loads: no staging registers, no staging VALU
//     work, and the weight image's 2304-byte blocks (one 32-column tile x four
//     K-blocks: codes, then scales) are copied verbatim;
//   - a stage holds 16 blocks (four groups of four); the four K waves of each
//     32-row half take one group each, so a stage costs one barrier per 16
//     blocks, and the next stage's loads are in flight during the current
//     stage's arithmetic (two LDS buffers);
//   - one 16-byte LDS read per lane gives one slot of the lane's weight
//     column for the group's four blocks (the image interleaves them), so a
//     wave reads its weight operands with two conflict-free reads per tile
//     and group; the activation rows sit in LDS with their 16-byte blocks
//     XOR-swizzled by row, so the operand reads of 32 rows spread over the
//     banks;
//   - v_mfma_i32_32x32x32_i8 per 32x32 tile and block, software-pipelined so
//     that each instruction's latency hides behind the previous tile's
//     epilogue;
//   - the partial sums of the four K waves are added through LDS in a fixed
//     order (wave 0, 1, 2, 3), so the result is bit-identical from run to run.
// Rows past M repeat the last row; blocks past K repeat the last block with
// weight scale 0 (the image pads them with scale 0), so they add exact zeros.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "operands.h"

namespace bpg {

namespace {

template <int TN_>
struct WideCfg {
    static constexpr int TN = TN_;                   // 32-column tiles per workgroup
    static constexpr int BM = 64, BN = 32 * TN;
    static constexpr int kThreads = 512;             // 2 row halves x 4 K waves
    static constexpr int kGroupBytes = 2304;         // image block: 32 columns x 4 K-blocks
    static constexpr int kTileBytes = 4 * kGroupBytes; // one tile's four groups of a stage
    // one stage in LDS: the image blocks [tile][group] verbatim, activation
    // codes [row][16 blocks] (16-byte blocks XOR-swizzled by row), row scales
    // [block][row] fp32
    static constexpr int kW = TN * kTileBytes;
    static constexpr int kA = BM * 16 * 16;
    static constexpr int kDa = 16 * BM * 4;
    static constexpr int kStage = kW + kA + kDa;
    static constexpr int kWLoads = kW / 1024;        // wave-wide 16-byte loads per stage
    static constexpr int kWPerWave = (kWLoads + 7) / 8;
    // final reduction: one tile at a time, [wave][16 regs][64 lanes], in the
    // first weight buffer
    static constexpr int kLdsRed = 8 * 16 * 64 * 4;
    static_assert(kW % 1024 == 0, "whole wave-wide loads");
    static_assert(kLdsRed <= kW, "reduction fits one weight buffer");
    static_assert(2 * kStage <= 160 * 1024, "LDS budget");
};

template <int TN>
__global__ __launch_bounds__(512, 1) void wide_kernel(GemmProblem p, int tiles_m)
{
    typedef WideCfg<TN> C;
    typedef Mfma<32> M;
    typedef M::Op Op;
    typedef M::Acc Acc;
    // two buffers, every region its own array: the compiler tells the direct
    // loads into one buffer from the reads of the other by the array they
    // address
    __shared__ __attribute__((aligned(16))) uint8_t w_lds0[C::kW];
    __shared__ __attribute__((aligned(16))) uint8_t w_lds1[C::kW];
    __shared__ __attribute__((aligned(16))) uint8_t a_lds0[C::kA];
    __shared__ __attribute__((aligned(16))) uint8_t a_lds1[C::kA];
    __shared__ __attribute__((aligned(16))) float d_lds0[C::kDa / 4];
    __shared__ __attribute__((aligned(16))) float d_lds1[C::kDa / 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;  // operand row / column, result column
    const int hk = lane >> 5; // operand K half, result row group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave & 3;  // K wave: group wk of every stage
    const int wm = wave >> 2; // row half

    const int B = (int)(p.k / 32); // the host limits K to 2^22
    const int NG = (B + 3) / 4;
    const int nst = (NG + 3) / 4;  // stages of four groups

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t row0 = (int64_t)(L % tiles_m) * C::BM;
    const int64_t col0 = (int64_t)(L / tiles_m) * C::BN;
    const int64_t rem = p.rows - 1 - row0;
    const int last_row = rem < C::BM - 1 ? (int)rem : C::BM - 1; // >= 0
    const int64_t arow = p.k / 2;

    // ---- direct-load sources of this lane, relative to the stage.  Every
    //      offset stays under 2^31 for K <= 2^22.
    const uint8_t *__restrict__ w_base = p.wcodes + (col0 >> 5) * NG * C::kGroupBytes;
    const uint8_t *__restrict__ a_base = p.codes + row0 * arow;
    const float *__restrict__ da_base = p.scales + row0 * B;
    // weights: chunk k = 1024 i + 16 lane of the stage's image copy is chunk
    // k % 2304 of group 4 st + gg of tile t
    uint32_t woff[C::kWPerWave];
    uint32_t wgg = 0; // 2 bits per load: the group within the stage
#pragma unroll
    for (int u = 0; u < C::kWPerWave; u++) {
        const int k = 64 * (wave + 8 * u) + lane; // 16-byte chunk index
        const int t = k / (C::kTileBytes / 16);
        const int r = k % (C::kTileBytes / 16);
        const int gg = r / (C::kGroupBytes / 16);
        woff[u] = (uint32_t)((t * NG + gg) * C::kGroupBytes + (r % (C::kGroupBytes / 16)) * 16);
        wgg |= (uint32_t)gg << (2 * u);
    }
    // activations: LDS chunk 64 i + lane = (row, j) holds block j ^ (row & 15)
    uint32_t aoff[2]; // row offset + block offset inside a full stage
    int ablk[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int ci = 64 * (wave + 8 * u) + lane;
        const int row = ci >> 4;
        ablk[u] = (ci & 15) ^ (row & 15);
        aoff[u] = (uint32_t)((row < last_row ? row : last_row) * arow + ablk[u] * 16);
    }
    // row scales: load i of a stage is block i, lane = row (byte offset)
    const uint32_t daoff = (uint32_t)((lane < last_row ? lane : last_row) * B * 4);

    // A stage whose 16 blocks all lie inside K (every stage but possibly the
    // last) needs neither masks nor clamps: every address is a uniform stage
    // base plus a fixed per-lane offset.  The last stage skips groups past
    // the image and repeats block B-1 for blocks past K.
    auto issue = [&](uint8_t *wl, uint8_t *al, float *dl, int st) {
        const int g0 = 4 * st;
        const uint8_t *wst = uniform(w_base + (size_t)g0 * C::kGroupBytes);
        const uint8_t *ast = uniform(a_base + (size_t)st * 256);
        const uint8_t *dst = uniform(reinterpret_cast<const uint8_t *>(da_base + 16 * st));
        if (16 * (st + 1) <= B) {
#pragma unroll
            for (int u = 0; u < C::kWPerWave; u++) {
                const int i = wave + 8 * u;
                if (i < C::kWLoads)
                    __builtin_amdgcn_global_load_lds((glb_void *)(wst + opaque(woff[u])),
                                                     (lds_void *)(wl + 1024 * i), 16, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 2; u++)
                __builtin_amdgcn_global_load_lds((glb_void *)(ast + opaque(aoff[u])),
                                                 (lds_void *)(al + 1024 * (wave + 8 * u)), 16, 0, 0);
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const int i = wave + 8 * u;
                __builtin_amdgcn_global_load_lds((glb_void *)(dst + 4 * i + opaque(daoff)),
                                                 (lds_void *)(dl + 64 * i), 4, 0, 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < C::kWPerWave; u++) {
                const int i = wave + 8 * u;
                if (i < C::kWLoads) {
                    const int gg = (int)((wgg >> (2 * u)) & 3);
                    // groups past the image belong to no K wave: not loaded
                    if (g0 + gg < NG)
                        __builtin_amdgcn_global_load_lds((glb_void *)(wst + opaque(woff[u])),
                                                         (lds_void *)(wl + 1024 * i), 16, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const int over = 16 * st + ablk[u] - (B - 1); // blocks past the last one
                const uint32_t off = aoff[u] - (over > 0 ? (uint32_t)over * 16 : 0u);
                __builtin_amdgcn_global_load_lds((glb_void *)(ast + opaque(off)),
                                                 (lds_void *)(al + 1024 * (wave + 8 * u)), 16, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const int i = wave + 8 * u;
                const int blk = 16 * st + i < B ? i : B - 1 - 16 * st;
                __builtin_amdgcn_global_load_lds((glb_void *)(dst + 4 * blk + opaque(daoff)),
                                                 (lds_void *)(dl + 64 * i), 4, 0, 0);
            }
        }
    };

    float acc[TN][16];
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            acc[j][r] = 0.0f;
    Acc magic;
#pragma unroll
    for (int r = 0; r < 16; r++)
        magic[r] = kMagicBits;

    // LDS read offsets of this lane, the same in every stage: activation
    // operand of block 4 wk + q (row wm*32 + c, bytes 8hk..8hk+7), row
    // scales of the lane's result rows for block 4 wk (+ 256 bytes per q)
    const int ar = wm * 32 + c;
    uint32_t a_rd[4];
#pragma unroll
    for (int q = 0; q < 4; q++)
        a_rd[q] = opaque((uint32_t)(ar * 256 + (((4 * wk + q) ^ (ar & 15)) * 16) + 8 * hk));
    const uint32_t d_rd = opaque((uint32_t)((4 * wk * 64 + wm * 32 + 4 * hk) * 4));

    // group wk of stage st, from one buffer
    auto compute = [&](const uint8_t *wl, const uint8_t *A, const float *Da, int st) {
        if (4 * st + wk >= NG)
            return; // uniform per wave
        // wave priority 1 for the stage's first two blocks, 0 for the last
        // two: a wave that has reached the second half yields issue slots to
        // one of its SIMD still in the first half, so the waves reach the
        // stage barrier closer together (3-6% faster on attn512-like shapes)
        __builtin_amdgcn_s_setprio(1);
        const uint8_t *W = wl + wk * C::kGroupBytes; // tile j at + j * kTileBytes
        // weight scales of the lane's column, four blocks per tile (fp16)
        uint2 hw[TN];
        // weight codes: slots 2hk and 2hk+1 of the lane's column, four blocks
        uint4 wr[TN][2];
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const uint8_t *Wt = W + j * C::kTileBytes;
            hw[j] = *reinterpret_cast<const uint2 *>(Wt + 2048 + ((c & 15) * 2 + (c >> 4)) * 8);
            wr[j][0] = *reinterpret_cast<const uint4 *>(Wt + ((2 * hk) * 32 + c) * 16);
            wr[j][1] = *reinterpret_cast<const uint4 *>(Wt + ((2 * hk + 1) * 32 + c) * 16);
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            if (q == 2)
                __builtin_amdgcn_s_setprio(0);
            const uint2 ad = *reinterpret_cast<const uint2 *>(A + a_rd[q]);
            Op a;
            a[0] = (int)act_lo(ad.x);
            a[1] = (int)act_lo(ad.y);
            a[2] = (int)act_hi(ad.x);
            a[3] = (int)act_hi(ad.y);
            float4 da[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++)
                da[r4] = *reinterpret_cast<const float4 *>(
                    reinterpret_cast<const uint8_t *>(Da) + d_rd + q * 256 + r4 * 32);
            // tile j's instruction is issued before tile j-1's epilogue
            Acc Dp;
            float dwp = 0.0f, nbp = 0.0f;
#pragma unroll
            for (int j = 0; j <= TN; j++) {
                Acc Dc;
                float dwc = 0.0f, nbc = 0.0f;
                if (j < TN) {
                    const uint32_t x = q == 0 ? wr[j][0].x : q == 1 ? wr[j][0].y : q == 2 ? wr[j][0].z : wr[j][0].w;
                    const uint32_t y = q == 0 ? wr[j][1].x : q == 1 ? wr[j][1].y : q == 2 ? wr[j][1].z : wr[j][1].w;
                    Op bo;
                    bo[0] = (int)q40_lo(x);
                    bo[1] = (int)q40_lo(y);
                    bo[2] = (int)q40_hi(x);
                    bo[3] = (int)q40_hi(y);
                    Dc = M::mma(a, bo, magic);
                    const uint32_t hd = q < 2 ? hw[j].x : hw[j].y;
                    // converted to fp32 here, so that the epilogue is plain
                    // fp32 FMAs (the compiler would otherwise fold the
                    // conversion into mixed-precision FMAs, which issue slower)
                    dwc = __uint_as_float(opaque(__float_as_uint(
                        half_bits_to_float((uint16_t)((q & 1) ? hd >> 16 : hd & 0xFFFFu)))));
                    nbc = -kMagic * dwc;
                }
                if (j > 0) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; r4++) {
                        const float dq[4] = {da[r4].x, da[r4].y, da[r4].z, da[r4].w};
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int r = 4 * r4 + e;
                            const float t = __builtin_fmaf(__int_as_float(Dp[r]), dwp, nbp);
                            acc[j - 1][r] = __builtin_fmaf(t, dq[e], acc[j - 1][r]);
                        }
                    }
                }
                if (j < TN) {
                    Dp = Dc;
                    dwp = dwc;
                    nbp = nbc;
                }
            }
        }
    };

    // s_waitcnt vmcnt(0): this wave's direct loads have reached LDS
    constexpr int kWaitLoads = 0x0F70;

    issue(w_lds0, a_lds0, d_lds0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitLoads);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst)
            issue(w_lds1, a_lds1, d_lds1, st + 1);
        compute(w_lds0, a_lds0, d_lds0, st);
        __builtin_amdgcn_s_waitcnt(kWaitLoads);
        __syncthreads();
        if (st + 1 < nst) {
            if (st + 2 < nst)
                issue(w_lds0, a_lds0, d_lds0, st + 2);
            compute(w_lds1, a_lds1, d_lds1, st + 1);
            __builtin_amdgcn_s_waitcnt(kWaitLoads);
            __syncthreads();
        }
    }

    // ---- fixed-order sum of the four K waves' partials (wk = 0, 1, 2, 3), two
    //      tiles at a time (one in each weight buffer); the widening factor
    //      256 is removed here.
    float *red0 = reinterpret_cast<float *>(w_lds0);
    float *red1 = reinterpret_cast<float *>(w_lds1);
    const int rows_valid = last_row + 1;
#pragma unroll
    for (int j0 = 0; j0 < TN; j0 += 2) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            red0[(wave * 16 + r) * 64 + lane] = acc[j0][r];
            if (j0 + 1 < TN)
                red1[(wave * 16 + r) * 64 + lane] = acc[j0 + 1][r];
        }
        __syncthreads();
        // wave wk of the half sums registers 4 wk .. 4 wk + 3 of both tiles
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            if (j0 + jj >= TN)
                continue;
            const float *red = jj == 0 ? red0 : red1;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 4 * wk + e;
                float v = red[((wm * 4 + 0) * 16 + r) * 64 + lane];
#pragma unroll
                for (int w = 1; w < 4; w++)
                    v += red[((wm * 4 + w) * 16 + r) * 64 + lane];
                const int rl = wm * 32 + M::out_row(hk, r);
                if (rl < rows_valid)
                    store_y(p, (row0 + rl) * p.ldy + col0 + (j0 + jj) * 32 + c, v * (1.0f / 256.0f));
            }
        }
        if (j0 + 2 < TN)
            __syncthreads();
    }
}

template <int TN>
hipError_t launch_tn(const GemmProblem &p, hipStream_t stream)
{
    const int tm = (int)((p.rows + 63) / 64), tn = (int)(p.n / (32 * TN));
    const int64_t grid = (int64_t)tm * tn;
    if (grid <= 0)
        return hipSuccess;
    wide_kernel<TN><<<dim3((unsigned)grid), 512, 0, stream>>>(p, tm);
    return hipGetLastError();
}

} // namespace

// 64 x 160 tiles (narrower tiles of this kernel lose to the strip kernel)
constexpr int kWideTN = 5;

bool wide_fits(const GemmProblem &p)
{
    return p.act_bits == 4 && p.experts == 1 && p.n % (32 * kWideTN) == 0 && p.rows > 0 &&
           (p.rows + 63) / 64 * (p.n / (32 * kWideTN)) < (int64_t)1 << 31;
}

hipError_t launch_wide(const GemmProblem &p, hipStream_t stream)
{
    return launch_tn<kWideTN>(p, stream);
}

} // namespace bpg
