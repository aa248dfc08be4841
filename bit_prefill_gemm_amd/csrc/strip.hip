// strip.hip -- the dense W4A4 product on 32-row strips (gfx950, 4- or
// 8-bit activation codes).
//
// "509 tokens a second of prompt: the Hadamard route ships", section "Why
// prompts are a matrix-unit problem": with hundreds of rows the product is
// matrix work, and on gfx950 its per-block scale epilogue (two fp32 VALU
// operations per output and block) is what bounds it.  This kernel keeps the
// operand layout of the wide kernel (wide.hip: image blocks copied verbatim
// into LDS by direct loads, activation blocks XOR-swizzled by row, row scales
// [block][row], one v_mfma_i32_32x32x32_i8 per 32x32 tile and block) but
// splits the work differently:
//   - a workgroup owns 32 rows x 128 columns and has four waves; wave t owns
//     32-column tile t over the whole of K, so no partial sums are added
//     across waves and every output is one wave's in-order accumulation;
//   - stages of 8 blocks with 4-bit codes, 4 with 8-bit codes (their rows
//     take twice the bytes), double-buffered (23 / 14 KB per stage), so
//     that three or more workgroups share a CU and run independently: one
//     computes while another waits at its barrier;
//   - three or more waves per SIMD, so each block's epilogue follows its
//     matrix instruction directly (other waves hide its latency); in the
//     last stage, code chunks of blocks past K are written as zeros (a zero
//     code makes the block product exactly zero whatever the weights), so
//     the arithmetic always covers whole stages.
// Rows past M repeat the last row (never stored).  Where 64 x 160 tiles fit
// and suit the shape, the wide kernel (wide.hip) is faster (fewer operand
// reads per product); elsewhere this kernel beats 64 x 128 and smaller tiles,
// and with 8-bit codes the tiled kernel (gemm.hip) wherever there are at
// least three strips per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "operands.h"

namespace bpg {

namespace {

template <int BITS_>
struct StripCfg {
    static constexpr int BITS = BITS_;              // activation code width
    static constexpr int TN = 4;                    // waves = 32-column tiles
    static constexpr int BM = 32, BN = 32 * TN;
    static constexpr int kThreads = 64 * TN;
    static constexpr int kOcc = 3;                  // workgroups per CU
    static constexpr int kWavesPerSimd = 3;         // (kOcc * 4 waves over 4 SIMDs)
    static constexpr int kGroupBytes = 2304;        // image block: 32 columns x 4 K-blocks
    static constexpr int kAB = BITS == 4 ? 16 : 32; // code bytes per row and block
    // blocks per stage: two groups for 4-bit codes, one for 8-bit (whose codes
    // take twice the bytes: three double-buffered workgroups must fit the LDS)
    static constexpr int kSB = BITS == 4 ? 8 : 4;
    static constexpr int kGroups = kSB / 4;
    static constexpr int kWTile = kGroups * kGroupBytes; // one tile's groups of a stage
    // one stage in LDS: image blocks [tile][group] verbatim, codes [row][8
    // 16-byte chunks] (chunks XOR-swizzled by row & 7), row scales [block][row]
    static constexpr int kW = TN * kWTile;
    static constexpr int kA = BM * kSB * kAB;
    static constexpr int kDa = kSB * BM * 4;
    static constexpr int kBuf = kW + kA + kDa;
    static constexpr int kWLoads = kW / 1024;       // wave-wide 16-byte weight loads
    static constexpr int kWPerWave = (kWLoads + TN - 1) / TN; // the last by some waves only
    static constexpr int kDaWaves = kDa / 256;      // waves with a row-scale load
    static constexpr float kUnscale = BITS == 4 ? 1.0f / 256.0f : 1.0f / 16.0f;
    static_assert(kW % 1024 == 0, "whole wave-wide weight loads");
    static_assert(kA == 4 * 1024 && kSB * kAB == 128, "one code load per wave, 128-byte rows");
    static_assert(kDa % 256 == 0 && kDaWaves <= TN, "row-scale loads");
    static_assert(kOcc * 2 * kBuf <= 160 * 1024, "LDS budget");
};

// Tile of workgroup w (of G = tm * tn): workgroups go to the 8 XCDs round
// robin (XCD w % 8, in the order w / 8 there).  XCD x owns a rectangle of
// the row tiles and column strips: part x / (8 / a) of a parts of the rows,
// part x % (8 / a) of 8 / a parts of the columns.  Inside it the workgroups
// walk row groups of rg tiles; in a row group, the column strips; in a strip,
// the group's rows.  The activation rows of a group stay in the XCD's L2
// while every strip of the rectangle streams past them.  Shapes that do not
// divide evenly keep the XCD-contiguous order of xcd_remap (column-major).
__device__ __forceinline__ void strip_tile(int w, int G, int tm, int tn, int a, int rg, int &rt,
                                           int &ct)
{
    const int b = 8 / a;
    if (G % 8 != 0 || a < 1 || 8 % a != 0 || tm % a != 0 || tn % b != 0 || rg < 1 ||
        (tm / a) % rg != 0) {
        const int L = xcd_remap(w, G);
        rt = L % tm;
        ct = L / tm;
        return;
    }
    const int x = w % 8, i = w / 8;
    const int R = tm / a, Cc = tn / b;
    const int g = i / (rg * Cc), rem = i - g * (rg * Cc);
    const int c = rem / rg, r = rem - c * rg;
    rt = (x / b) * R + g * rg + r;
    ct = (x % b) * Cc + c;
}

// (the second bound is the minimum number of waves per SIMD)
template <int BITS>
__global__ __launch_bounds__(StripCfg<BITS>::kThreads, StripCfg<BITS>::kWavesPerSimd) void
strip_kernel(GemmProblem p, int tiles_m, int parts_m, int row_group)
{
    typedef StripCfg<BITS> C;
    constexpr int TN = C::TN;
    typedef Mfma<32> M;
    typedef M::Op Op;
    typedef M::Acc Acc;
    // two stage buffers, each its own array (the compiler tells the direct
    // loads into one from the reads of the other by the array they address)
    __shared__ __attribute__((aligned(16))) uint8_t buf0[C::kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[C::kBuf];
    constexpr int kG = C::kGroups;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;  // operand row / column, result column
    const int hk = lane >> 5; // operand K half, result row group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // = the wave's tile

    const int B = (int)(p.k / 32); // the host limits K to 2^22
    const int NG = (B + 3) / 4;
    const int nst = (NG + kG - 1) / kG; // stages of kG groups
    const int64_t arow = p.k / 32 * C::kAB;

    int rt, ct;
    strip_tile(blockIdx.x, gridDim.x, tiles_m, (int)(p.n / C::BN), parts_m, row_group, rt, ct);
    const int64_t row0 = (int64_t)rt * C::BM;
    const int64_t col0 = (int64_t)ct * C::BN;
    const int64_t rem = p.rows - 1 - row0;
    const int last_row = rem < C::BM - 1 ? (int)rem : C::BM - 1; // >= 0

    // ---- direct-load sources of this lane, relative to the stage (every
    //      offset stays under 2^31 for K <= 2^22)
    const uint8_t *__restrict__ w_base = p.wcodes + (col0 >> 5) * NG * C::kGroupBytes;
    const uint8_t *__restrict__ a_base = p.codes + row0 * arow;
    const float *__restrict__ da_base = p.scales + row0 * B;
    // weights: byte b of a stage's copy is byte b % 2304 of group 2 st + gg
    // of tile t; 16-byte loads i = wave + TN u < kWLoads, b = 1024 i + 16 lane
    uint32_t woff[C::kWPerWave];
    uint32_t wgg = 0; // bit u: the load's group within the stage
#pragma unroll
    for (int u = 0; u < C::kWPerWave; u++) {
        const int i = wave + TN * u;
        const int b = 1024 * (i < C::kWLoads ? i : 0) + 16 * lane;
        const int t = b / C::kWTile;
        const int r = b % C::kWTile;
        const int gg = r / C::kGroupBytes;
        woff[u] = (uint32_t)((t * NG + gg) * C::kGroupBytes + r % C::kGroupBytes);
        wgg |= (uint32_t)gg << u;
    }
    // codes: wave w loads chunks 64 w + lane = (row 8 w + lane / 8, slot
    // lane % 8), slot j holding chunk j ^ (row & 7) of the row's 128 bytes
    const int arow_l = 8 * wave + (lane >> 3);
    const int achunk = (lane & 7) ^ (arow_l & 7);
    const int ablk = achunk / (C::kAB / 16);
    const uint32_t aoff =
        (uint32_t)((arow_l < last_row ? arow_l : last_row) * arow + achunk * 16);
    // row scales: wave w loads blocks 2w, 2w+1 (lane / 32) of rows lane % 32
    const uint32_t daoff =
        (uint32_t)(((c < last_row ? c : last_row) * B + hk) * 4);

    auto issue = [&](uint8_t *buf, int st) __attribute__((always_inline)) {
        const int g0 = kG * st;
        const uint8_t *wst = uniform(w_base + (size_t)g0 * C::kGroupBytes);
        const uint8_t *ast = uniform(a_base + (size_t)st * (C::kSB * C::kAB));
        const uint8_t *dst = uniform(reinterpret_cast<const uint8_t *>(da_base + C::kSB * st));
        uint8_t *wl = buf;
        uint8_t *al = buf + C::kW;
        uint8_t *dl = buf + C::kW + C::kA;
        const bool tail = C::kSB * (st + 1) > B;
        const bool over_g = kG == 2 && g0 + 1 >= NG; // the stage's second group is past the image
#pragma unroll
        for (int u = 0; u < C::kWPerWave; u++) {
            const int i = wave + TN * u;
            if (i < C::kWLoads) {
                // in the last stage a group past the image repeats the one before
                const uint32_t o =
                    woff[u] - (tail && over_g && ((wgg >> u) & 1) ? (uint32_t)C::kGroupBytes : 0u);
                __builtin_amdgcn_global_load_lds((glb_void *)(wst + opaque(o)),
                                                 (lds_void *)(wl + 1024 * i), 16, 0, 0);
            }
        }
        uint8_t *adst = al + 1024 * wave;
        if (!tail || C::kSB * st + ablk < B)
            __builtin_amdgcn_global_load_lds((glb_void *)(ast + opaque(aoff)), (lds_void *)adst,
                                             16, 0, 0);
        else
            *reinterpret_cast<uint4 *>(adst + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
        // blocks 2 wave + hk of the stage; past K, block B-1
        if (wave < C::kDaWaves) {
            const int blk =
                C::kSB * st + 2 * wave + hk < B ? 2 * wave : B - 1 - C::kSB * st - hk;
            __builtin_amdgcn_global_load_lds((glb_void *)(dst + opaque(daoff + 4 * blk)),
                                             (lds_void *)(dl + 256 * wave), 4, 0, 0);
        }
    };

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; r++)
        acc[r] = 0.0f;
    Acc magic;
#pragma unroll
    for (int r = 0; r < 16; r++)
        magic[r] = kMagicBits;

    // LDS read offsets inside a buffer (each read address is its array plus
    // one integer offset: longer address chains lose the array's identity,
    // and the compiler then waits for the direct loads into the other buffer
    // before the read).  Weight slots 2hk, 2hk+1 of the lane's column and its
    // fp16 scales in group g of the wave's tile (+ 2304 g); codes of row c:
    // 4-bit, bytes 8hk..8hk+7 of block q (slot q ^ (c & 7)), 8-bit, bytes
    // 8hk..8hk+7 of each 16-byte half of block q (slots 2q ^ (c & 7) and
    // (2q + 1) ^ (c & 7)): the K values 8hk..8hk+7 and 16+8hk..16+8hk+7 that
    // the weight operand holds; row scales of the lane's result rows
    // 4hk + 8 r4 .. + 3 of block q (+ 128 q).
    const uint32_t w_rd = opaque((uint32_t)(wave * C::kWTile + ((2 * hk) * 32 + c) * 16));
    const uint32_t hw_rd =
        opaque((uint32_t)(wave * C::kWTile + 2048 + ((c & 15) * 2 + (c >> 4)) * 8));
    const uint32_t a_rd = opaque((uint32_t)(C::kW + c * 128 + 8 * hk));
    const uint32_t d_rd = opaque((uint32_t)(C::kW + C::kA + 4 * hk * 4));
    const int csw = c & 7;

    // the wave's tile over the stage's eight blocks (each block's epilogue
    // right after its matrix instruction: the other waves of the SIMD hide the
    // instruction's latency)
    auto compute = [&](const uint8_t *buf) __attribute__((always_inline)) {
        uint4 wr[kG][2];
        uint2 hw[kG];
#pragma unroll
        for (int g = 0; g < kG; g++) {
            wr[g][0] = *reinterpret_cast<const uint4 *>(buf + (w_rd + g * C::kGroupBytes));
            wr[g][1] = *reinterpret_cast<const uint4 *>(buf + (w_rd + g * C::kGroupBytes + 512));
            hw[g] = *reinterpret_cast<const uint2 *>(buf + (hw_rd + g * C::kGroupBytes));
        }
#pragma unroll
        for (int q = 0; q < C::kSB; q++) {
            Op a;
            if (BITS == 4) {
                const uint2 ad = *reinterpret_cast<const uint2 *>(
                    buf + (a_rd + (uint32_t)((q ^ csw) * 16)));
                a[0] = (int)act_lo(ad.x);
                a[1] = (int)act_lo(ad.y);
                a[2] = (int)act_hi(ad.x);
                a[3] = (int)act_hi(ad.y);
            } else {
                const uint2 lo = *reinterpret_cast<const uint2 *>(
                    buf + (a_rd + (uint32_t)(((2 * q) ^ csw) * 16)));
                const uint2 hi = *reinterpret_cast<const uint2 *>(
                    buf + (a_rd + (uint32_t)(((2 * q + 1) ^ csw) * 16)));
                a[0] = (int)lo.x;
                a[1] = (int)lo.y;
                a[2] = (int)hi.x;
                a[3] = (int)hi.y;
            }
            float4 da[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++)
                da[r4] = *reinterpret_cast<const float4 *>(buf + (d_rd + q * 128 + r4 * 32));
            const int g = q >> 2, qq = q & 3;
            const uint32_t x = qq == 0 ? wr[g][0].x : qq == 1 ? wr[g][0].y : qq == 2 ? wr[g][0].z : wr[g][0].w;
            const uint32_t y = qq == 0 ? wr[g][1].x : qq == 1 ? wr[g][1].y : qq == 2 ? wr[g][1].z : wr[g][1].w;
            Op bo;
            bo[0] = (int)q40_lo(x);
            bo[1] = (int)q40_lo(y);
            bo[2] = (int)q40_hi(x);
            bo[3] = (int)q40_hi(y);
            const Acc D = M::mma(a, bo, magic);
            const uint32_t hd = qq < 2 ? hw[g].x : hw[g].y;
            // converted here, so that the epilogue is plain fp32 FMAs
            const float dw = __uint_as_float(opaque(__float_as_uint(
                half_bits_to_float((uint16_t)((qq & 1) ? hd >> 16 : hd & 0xFFFFu)))));
            const float nb = -kMagic * dw;
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                const float dq[4] = {da[r4].x, da[r4].y, da[r4].z, da[r4].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * r4 + e;
                    const float t = __builtin_fmaf(__int_as_float(D[r]), dw, nb);
                    acc[r] = __builtin_fmaf(t, dq[e], acc[r]);
                }
            }
            // one block at a time (the registers must allow the waves per
            // SIMD above)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // s_waitcnt vmcnt(0): this wave's direct loads have reached LDS
    constexpr int kWaitLoads = 0x0F70;

    issue(buf0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitLoads);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst)
            issue(buf1, st + 1);
        compute(buf0);
        __builtin_amdgcn_s_waitcnt(kWaitLoads);
        __syncthreads();
        if (st + 1 < nst) {
            if (st + 2 < nst)
                issue(buf0, st + 2);
            compute(buf1);
            __builtin_amdgcn_s_waitcnt(kWaitLoads);
            __syncthreads();
        }
    }

    // the wave's tile; the widening factor (256, 8-bit codes 16) is removed here
    const int64_t y0 = (row0 + 4 * hk) * p.ldy + col0 + wave * 32 + c;
    const int lim = last_row + 1 - 4 * hk; // rows of this lane's group that hold data
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int ro = 8 * (r >> 2) + (r & 3);
        if (ro < lim)
            store_y(p, y0 + (int64_t)ro * p.ldy, acc[r] * C::kUnscale);
    }
}

} // namespace

bool strip_fits(const GemmProblem &p)
{
    return (p.act_bits == 4 || p.act_bits == 8) && p.experts == 1 && p.n % 128 == 0 &&
           p.rows > 0 && (p.rows + 31) / 32 * (p.n / 128) < (int64_t)1 << 31;
}

// The XCD rectangles of strip_tile: the fewest row parts a (1, 2, 4, 8)
// whose activation slice (codes and fp32 scales of tm / a row tiles) stays
// within 3 MB of an XCD's 4 MB L2 while the rectangle's weight strips stream
// past it; every XCD then reads its slice once and each of its strips once.
// Measured on 1024 x 5120 x 17408 (FETCH_SIZE per launch): 4-bit 174 -> 123
// MB (a = 2 against the column-only split), 8-bit 620 -> 215 MB.
void strip_order(const GemmProblem &p, int tm, int tn, int &a, int &rg)
{
    const int64_t row_bytes = p.k * p.act_bits / 8 + p.k / 8; // codes + scales of one row
    const int64_t act = (int64_t)tm * StripCfg<4>::BM * row_bytes;
    for (a = 1; a < 8; a *= 2)
        if (act / a <= ((int64_t)3 << 20) && tm % a == 0 && tn % (8 / a) == 0)
            break;
    if (tm % a != 0 || tn % (8 / a) != 0)
        a = 1; // strip_tile then keeps the XCD-contiguous order
    rg = tm / a > 0 ? tm / a : 1;
}

hipError_t launch_strip(const GemmProblem &p, hipStream_t stream)
{
    const int tm = (int)((p.rows + 31) / 32), tn = (int)(p.n / 128);
    const int64_t grid = (int64_t)tm * tn;
    if (grid <= 0)
        return hipSuccess;
    int a = 1, rg = tm;
    strip_order(p, tm, tn, a, rg);
    if (p.act_bits == 4)
        strip_kernel<4><<<dim3((unsigned)grid), StripCfg<4>::kThreads, 0, stream>>>(p, tm, a, rg);
    else
        strip_kernel<8><<<dim3((unsigned)grid), StripCfg<8>::kThreads, 0, stream>>>(p, tm, a, rg);
    return hipGetLastError();
}

} // namespace bpg
