// gemm.hip -- W4A4 / W4A8 products on CDNA4 integer matrix cores (gfx950).
//
// "509 tokens a second of prompt: the Hadamard route ships", section "Why
// prompts are a matrix-unit problem": prompts are a matrix-unit workload; a
// Q4_0 code u means u-8, which is the code with its top bit flipped read as a
// 4-bit two's-complement number, so the kernel reads Q4_0 nibbles bit for bit.
// gfx950 has no int4 matrix instruction: both operands are widened to int8 in
// registers, and every 32-value block is one integer matrix instruction per
// output tile with K = 32 (so each result is exactly one block sum):
// v_mfma_i32_32x32x32_i8 (32x32 tiles, the double-rate gfx950 form) for the
// wide shapes, v_mfma_i32_16x16x32_i8 (16x16 tiles) for short or ragged ones.
//
// Per K-block b the kernel needs y[m][n] += da[m][b] * dw[n][b] * S[m][n][b]
// with S the exact int32 block dot product:
//   - operands are widened as 16*value (the nibble in the top half of a byte),
//     so the instruction returns 256*S (8-bit activations: 16*S); the power
//     of two is removed once, when the output is stored;
//   - the accumulator input is 0x4B400000 (1.5*2^23 as fp32), so the int32
//     result read as fp32 is exactly 12582912 + 256*S (|256*S| < 2^22);
//   - t = fma(F, dw, -12582912*dw) = 256*S*dw (the constant product is exact:
//     dw is an fp16 value, 11 significant bits), then acc = fma(t, da, acc).
// Two fp32 VALU operations per (m, n, b) and no integer conversion.  Packed
// fp32 is not used, so that epilogue, not the matrix core, bounds the kernel.
//
// Work split: a workgroup owns a BM x BN output tile split among WM x WN wave
// groups; the WK waves of a group each take every WK-th block of a stage and
// keep partial sums of the group's tile, which are added in a fixed order
// (wave 0, 1, ...) through LDS at the end, so the result is bit-identical from
// run to run.  Operands are staged through LDS, KC blocks per stage, double
// buffered, with the next stage's global loads in flight during the current
// stage's arithmetic.
//
// The same main loop also runs in block-sum mode (exact int32 S for parity
// checks) and in grouped mode (rows sorted by expert, ragged row ranges).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "operands.h"

namespace bpg {

namespace {

enum Mode { kGemm = 0, kGrouped = 1, kSums = 2 };

// MF: matrix instruction tile (16 or 32).  Wave layout: WM x WN x WK waves;
// wave (wm, wn, wk) owns the TM x TN tiles of MF x MF at row tile wm*TM and
// column tile wn*TN of the workgroup tile, and every WK-th block of a stage.
template <int BITS_, int MF_, int TM_, int TN_, int WM_, int WN_, int WK_, int KC_>
struct Cfg {
    static constexpr int BITS = BITS_, MF = MF_, TM = TM_, TN = TN_, KC = KC_;
    static constexpr int WM = WM_, WN = WN_, WK = WK_;
    static constexpr int kWaves = WM * WN * WK;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = MF * TM * WM, BN = MF * TN * WN;
    static constexpr int kRegs = MF * MF / 64;        // output registers per tile and lane
    static constexpr int kAB = BITS == 4 ? 16 : 32;   // code bytes per (row, block)
    static constexpr int kShift = BITS == 4 ? 8 : 4;  // log2 of the operand widening
    // one stage in LDS: A codes [KC][BM][kAB], W codes [KC][BN][16],
    // row scales [KC][BM] fp32, column scales [KC][BN] (dw, -12582912*dw)
    static constexpr int kLdsA = KC * BM * kAB;
    static constexpr int kLdsW = KC * BN * 16;
    static constexpr int kLdsDa = KC * BM * 4;
    static constexpr int kLdsDw = KC * BN * 8;
    static constexpr int kStage = kLdsA + kLdsW + kLdsDa + kLdsDw;
    static constexpr int kTiles = TM * TN; // per wave
    // final reduction: every wave parks the partial sums of up to kRedTiles
    // of its tiles at a time ([group][wk][tile][kRegs][64 lanes] fp32)
    static constexpr int kRedCap = MF == 16 ? 16 : 4;
    static constexpr int kRedTiles = kTiles < kRedCap ? kTiles : kRedCap;
    static constexpr int kLdsRed = kWaves * kRedTiles * kRegs * 64 * 4;
    static constexpr int kLds = 2 * kStage > kLdsRed ? 2 * kStage : kLdsRed;
    // 16-byte global chunks per stage and per thread
    static constexpr int kChA = BM * KC * (kAB / 16);
    static constexpr int kChW = BN * KC;
    static constexpr int kPtA = (kChA + kThreads - 1) / kThreads;
    static constexpr int kPtW = (kChW + kThreads - 1) / kThreads;
    static constexpr int kPtDa = (BM * KC + kThreads - 1) / kThreads;
    static constexpr int kChDw = BN * KC / 4; // 8-byte chunks: four blocks' scales
    static constexpr int kPtDw = (kChDw + kThreads - 1) / kThreads;
    static constexpr int kOcc = kThreads >= 512 ? 1 : 2; // workgroups per CU aimed at
    static_assert(MF == 16 || MF == 32, "matrix tile");
    static_assert(KC % WK == 0 && KC <= 16, "K split and swizzle range");
    static_assert(KC % 4 == 0, "stages hold whole groups of four blocks");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

// LDS slot of activation row `r` of block `kc`: the low four bits are
// XOR-swizzled so that both the staging writes (8 consecutive lanes write the
// 8 blocks of one row, 16 lanes two rows) and the operand reads (consecutive
// rows of one block) spread over the banks.  A bijection inside every aligned
// group of 16.  Weight columns need none: their staging writes one dword
// slot of 16 consecutive columns at a time.
__device__ __forceinline__ int swz(int r, int kc) { return r ^ kc ^ ((r & 1) << 3); }

// Grouped tiling: expert e owns ceil(rows_e / BM) consecutive row slots.  Find
// the expert and the row range of `slot` with a scan over the clamped offsets
// done by every wave on its own (no LDS, no barrier; each wave reaches the
// same answer): lanes take four experts each, 256 experts per pass.  Returns
// false (uniformly) if the slot lies beyond the last tile.  Every row range
// returned lies inside [0, rows).
template <int BM>
__device__ bool grouped_slot(const int32_t *__restrict__ off, int64_t experts, int64_t rows64,
                             int slot, int64_t &row0, int64_t &row_end, int64_t &expert)
{
    const int lane = threadIdx.x & 63;
    const int rows = (int)rows64; // the host limits rows to 2^31 - 1
    int64_t carry = 0;            // slots of the experts before this pass
    for (int64_t base = 0; base < experts; base += 256) {
        int a[4], b[4];
        int cnt[4], lsum = 0;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int64_t e = base + 4 * lane + u;
            a[u] = b[u] = 0;
            cnt[u] = 0;
            if (e < experts) {
                a[u] = min(max(off[e], 0), rows);
                b[u] = min(max(off[e + 1], 0), rows);
                if (b[u] > a[u])
                    cnt[u] = (int)(((unsigned)(b[u] - a[u]) + BM - 1) / BM);
            }
            lsum += cnt[u];
        }
        int incl = lsum; // inclusive scan of the lanes' counts
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d)
                incl += v;
        }
        const int64_t rel = slot - carry;
        const int excl = incl - lsum;
        const uint64_t owner = __ballot(rel >= excl && rel < incl);
        if (owner != 0) {
            const int src = __ffsll((unsigned long long)owner) - 1;
            // the owning lane walks its four experts
            int64_t r0 = 0, r1 = 0, ex = 0;
            int64_t s = rel - excl;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                if (s >= 0 && s < cnt[u]) {
                    r0 = a[u] + s * BM;
                    r1 = b[u];
                    ex = base + 4 * lane + u;
                }
                s -= cnt[u];
            }
            row0 = __shfl(r0, src);
            row_end = __shfl(r1, src);
            expert = __shfl(ex, src);
            return true;
        }
        carry += __shfl(incl, 63);
    }
    return false;
}

// f(integral_constant<int, n>) for the runtime count 1 <= n <= N.
template <int N, class F>
__device__ __forceinline__ void with_count(int n, F &&f)
{
    if constexpr (N == 1) {
        f(std::integral_constant<int, 1>{});
    } else {
        if (n >= N)
            f(std::integral_constant<int, N>{});
        else
            with_count<N - 1>(n, f);
    }
}

template <class C, int MODE>
__global__ __launch_bounds__(C::kThreads, C::kOcc) void w4a4_kernel(GemmProblem p, int tiles_m,
                                                              int tiles_n, int tm0, int tn0)
{
    constexpr int BM = C::BM, BN = C::BN, KC = C::KC, TM = C::TM, TN = C::TN, MF = C::MF;
    constexpr int NT = C::kThreads, kAB = C::kAB, WK = C::WK, RG = C::kRegs;
    typedef Mfma<MF> M;
    typedef typename M::Op Op;
    typedef typename M::Acc Acc;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rc = M::rc(lane); // operand row / column, result column, inside a tile
    const int g = M::kg(lane);  // operand K group, result row group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave % C::WK;
    const int wn = (wave / C::WK) % C::WN;
    const int wm = wave / (C::WK * C::WN);
    const int grp = wm * C::WN + wn; // waves of one group share tiles, split K

    const int B = (int)(p.k / 32); // the host limits K to 2^22
    const int NG = (B + 3) / 4;     // groups of four blocks in the weight image
    const int64_t ntiles32 = p.n / 32;

    // ---- the tile of this workgroup
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    int64_t row0, row_end, col0, expert;
    if (MODE == kGrouped) {
        const int slot = L / tiles_n;
        col0 = (int64_t)(L % tiles_n) * BN;
        if (!grouped_slot<BM>(p.offsets, p.experts, p.rows, slot, row0, row_end, expert))
            return; // uniform across the workgroup
    } else {
        row0 = (int64_t)(tm0 + L % tiles_m) * BM;
        col0 = (int64_t)(tn0 + L / tiles_m) * BN;
        row_end = p.rows;
        expert = MODE == kSums ? p.expert : 0;
    }
    const int64_t arow_bytes = p.k * kAB / 32;
    const int64_t ct0 = col0 >> 5; // first 32-column image tile touched by this tile

    // ---- staging addresses, computed once.  Global reads are coalesced
    //      (consecutive threads read consecutive blocks of a row, or
    //      consecutive columns); LDS slots are swizzled (swz).  Rows past
    //      row_end are clamped to the last valid row: their values only reach
    //      output rows that are never stored.
    // (every offset below stays under 2^31 for K <= 2^22)
    // Grouped rows may gather their activation rows through p.row_ids (the
    // offsets are then taken from row 0; the host keeps src_rows * row bytes
    // under 2^31).
    const bool gather = MODE == kGrouped && p.row_ids != nullptr;
    auto src_row = [&](int rrow) -> int64_t {
        if (!gather)
            return rrow;
        const int64_t r = p.row_ids[row0 + rrow];
        return r < 0 ? 0 : (r >= p.src_rows ? p.src_rows - 1 : r);
    };
    const uint8_t *__restrict__ a_base0 = p.codes + (gather ? 0 : row0) * arow_bytes;
    // weight image: 2304-byte blocks per (expert, 32-column tile, group of
    // four K-blocks): 2048 code bytes, then 128 fp16 scales (p.wscales points
    // at the first block's scales)
    const uint8_t *__restrict__ w_base0 = p.wcodes + (expert * ntiles32 + ct0) * NG * 2304;
    const float *__restrict__ da_base0 = p.scales + (gather ? 0 : row0) * B;
    const uint16_t *__restrict__ dw_base0 = p.wscales + (expert * ntiles32 + ct0) * NG * 1152;
    const int last_row = (int)(row_end - 1 - row0); // >= 0

    uint32_t oa[C::kPtA], la[C::kPtA], ow[C::kPtW], lw[C::kPtW];
    uint32_t oda[C::kPtDa], lda_[C::kPtDa], odw[C::kPtDw], ldw_[C::kPtDw];
    int8_t kca[C::kPtA], kcw[C::kPtW], kcda[C::kPtDa], kcdw[C::kPtDw]; // first block of each chunk
#pragma unroll
    for (int i = 0; i < C::kPtA; i++) {
        const int c = tid + i * NT;
        const int cc = c < C::kChA ? c : 0;
        const int row = cc / (KC * (kAB / 16));
        const int rem = cc % (KC * (kAB / 16));
        const int kc = rem / (kAB / 16), part = rem % (kAB / 16);
        const int rrow = row < last_row ? row : last_row;
        oa[i] = (uint32_t)(src_row(rrow) * arow_bytes + kc * kAB + part * 16);
        const int srow = swz(row, kc);
        // 8-bit codes: the two 16-byte halves of a row block swap places on
        // every other group of 8 rows (reads of 16 rows then avoid conflicts)
        const int slot = kAB == 32 ? (part ^ ((srow >> 3) & 1)) : 0;
        la[i] = (uint32_t)((kc * BM + srow) * kAB + slot * 16);
        kca[i] = (int8_t)(c < C::kChA ? kc : 127);
    }
#pragma unroll
    for (int i = 0; i < C::kPtW; i++) {
        const int c = tid + i * NT;
        // chunk: slot s of column col for the four blocks of group gs
        const int cc = c < C::kChW ? c : 0;
        const int s = cc & 3, col = (cc >> 2) % BN, gs = (cc >> 2) / BN;
        const int64_t gcol = col0 + col;
        ow[i] = (uint32_t)((((gcol >> 5) - ct0) * NG + gs) * 2304 + (s * 32 + (gcol & 31)) * 16);
        lw[i] = (uint32_t)((4 * gs * BN + col) * 16 + 4 * s); // block 4*gs; + q*BN*16 for 4*gs+q
        kcw[i] = (int8_t)(c < C::kChW ? 4 * gs : 127);
    }
#pragma unroll
    for (int i = 0; i < C::kPtDa; i++) {
        const int c = tid + i * NT;
        const int cc = c < BM * KC ? c : 0;
        const int kc = cc / BM, row = cc % BM;
        const int rrow = row < last_row ? row : last_row;
        oda[i] = (uint32_t)(src_row(rrow) * B + kc);
        lda_[i] = (uint32_t)(kc * BM + row);
        kcda[i] = (int8_t)(c < BM * KC ? kc : 127);
    }
#pragma unroll
    for (int i = 0; i < C::kPtDw; i++) {
        const int c = tid + i * NT;
        // chunk: the scales of column col for the four blocks of group gs
        const int cc = c < C::kChDw ? c : 0;
        const int gs = cc / BN, col = cc % BN;
        const int64_t gcol = col0 + col;
        const int c32 = (int)(gcol & 31);
        odw[i] = (uint32_t)((((gcol >> 5) - ct0) * NG + gs) * 1152 + ((c32 % 16) * 2 + c32 / 16) * 4);
        ldw_[i] = (uint32_t)(4 * gs * BN + col);
        kcdw[i] = (int8_t)(c < C::kChDw ? 4 * gs : 127);
    }

    // ---- global -> registers -> LDS staging of one stage (KC blocks)
    uint4 ra[C::kPtA], rw[C::kPtW];
    float rda[C::kPtDa];
    uint2 rdw[C::kPtDw];

    // Chunk i of a thread exists for every thread when (i+1)*NT <= count;
    // only the last chunk of a region can exist for some threads only.
#define BPG_CHUNK_OK(i, count) ((((i) + 1) * NT <= (count)) || (tid + (i) * NT < (count)))
    // Full stages read every chunk; the last, partial stage skips blocks past K.
    // A thread whose last chunk does not exist reads chunk 0 instead (its
    // offsets were set so) and never stores it: loads without a lane mask keep
    // the waits before the stores simple.
    auto load_stage = [&](int kb0, auto full_tag) {
        constexpr bool full = decltype(full_tag)::value;
        const int kv = full ? KC : B - kb0;
        const uint8_t *ab = a_base0 + kb0 * kAB;
        const uint8_t *wb = w_base0 + kb0 * 576;   // kb0 / 4 groups of 2304 bytes
        const float *dab = da_base0 + kb0;
        const uint16_t *dwb = dw_base0 + kb0 * 288; // kb0 / 4 groups, 1152 fp16 apart
#pragma unroll
        for (int i = 0; i < C::kPtA; i++)
            ra[i] = (full || kca[i] < kv)
                        ? *reinterpret_cast<const uint4 *>(ab + oa[i]) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < C::kPtW; i++)
            rw[i] = (full || kcw[i] < kv)
                        ? *reinterpret_cast<const uint4 *>(wb + ow[i]) : make_uint4(0, 0, 0, 0);
        if (MODE != kSums) { // block sums never read scales
#pragma unroll
            for (int i = 0; i < C::kPtDa; i++)
                rda[i] = (full || kcda[i] < kv) ? dab[oda[i]] : 0.0f;
#pragma unroll
            for (int i = 0; i < C::kPtDw; i++)
                rdw[i] = (full || kcdw[i] < kv)
                             ? *reinterpret_cast<const uint2 *>(dwb + odw[i]) : make_uint2(0, 0);
        }
    };

    auto store_stage = [&](uint8_t *A) {
        uint8_t *W = A + C::kLdsA;
        float *Da = reinterpret_cast<float *>(W + C::kLdsW);
        float2 *Dw = reinterpret_cast<float2 *>(W + C::kLdsW + C::kLdsDa);
#pragma unroll
        for (int i = 0; i < C::kPtA; i++)
            if (BPG_CHUNK_OK(i, C::kChA))
                *reinterpret_cast<uint4 *>(A + la[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < C::kPtW; i++)
            if (BPG_CHUNK_OK(i, C::kChW)) {
                const uint32_t v[4] = {rw[i].x, rw[i].y, rw[i].z, rw[i].w};
#pragma unroll
                for (int q = 0; q < 4; q++)
                    *reinterpret_cast<uint32_t *>(W + lw[i] + q * BN * 16) = v[q];
            }
        if (MODE != kSums) {
#pragma unroll
            for (int i = 0; i < C::kPtDa; i++)
                if (BPG_CHUNK_OK(i, BM * KC))
                    Da[lda_[i]] = rda[i];
#pragma unroll
            for (int i = 0; i < C::kPtDw; i++)
                if (BPG_CHUNK_OK(i, C::kChDw)) {
                    const uint16_t h[4] = {(uint16_t)(rdw[i].x & 0xFFFFu), (uint16_t)(rdw[i].x >> 16),
                                           (uint16_t)(rdw[i].y & 0xFFFFu), (uint16_t)(rdw[i].y >> 16)};
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const float dw = half_bits_to_float(h[q]);
                        Dw[ldw_[i] + q * BN] = make_float2(dw, -kMagic * dw);
                    }
                }
        }
    };
#undef BPG_CHUNK_OK

    // rows of each of this wave's row tiles that hold data (uniform per wave)
    int vrows[TM];
    int nact = 0; // row tiles with data: the first nact
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int64_t v = row_end - (row0 + (int64_t)(wm * TM + i) * MF);
        vrows[i] = v < 0 ? 0 : (v > MF ? MF : (int)v);
        nact += vrows[i] > 0;
    }
    // Grouped slots often hold fewer rows than the tile (an expert's rows):
    // the row tiles without data skip their products and epilogues.  The
    // stage arithmetic is compiled once per count of active row tiles and
    // chosen per stage (a uniform branch), so the tile loops stay free of
    // branches.  The dense shapes compute every tile (padded rows are never
    // stored).

    float acc[TM][TN][RG];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < RG; r++)
                acc[i][j][r] = 0.0f;

    Acc magic;
#pragma unroll
    for (int r = 0; r < RG; r++)
        magic[r] = kMagicBits;

    // matrix operands of row `srow` / column `scol` (LDS slots) of block kc
    auto load_a = [&](const uint8_t *A, int kc, int srow) -> Op {
        const uint8_t *rowp = A + (kc * BM + srow) * kAB;
        if constexpr (MF == 16) {
            if constexpr (kAB == 16) {
                const uint32_t d = *reinterpret_cast<const uint32_t *>(rowp + 4 * g);
                return pack2(act_lo(d), act_hi(d));
            } else {
                const int sw = (srow >> 3) & 1;
                const uint32_t lo = *reinterpret_cast<const uint32_t *>(rowp + sw * 16 + 4 * g);
                const uint32_t hi = *reinterpret_cast<const uint32_t *>(rowp + (sw ^ 1) * 16 + 4 * g);
                return pack2(lo, hi);
            }
        } else {
            Op o;
            if constexpr (kAB == 16) {
                const uint2 d = *reinterpret_cast<const uint2 *>(rowp + 8 * g);
                o[0] = (int)act_lo(d.x);
                o[1] = (int)act_lo(d.y);
                o[2] = (int)act_hi(d.x);
                o[3] = (int)act_hi(d.y);
            } else {
                const int sw = (srow >> 3) & 1;
                const uint2 lo = *reinterpret_cast<const uint2 *>(rowp + sw * 16 + 8 * g);
                const uint2 hi = *reinterpret_cast<const uint2 *>(rowp + (sw ^ 1) * 16 + 8 * g);
                o[0] = (int)lo.x;
                o[1] = (int)lo.y;
                o[2] = (int)hi.x;
                o[3] = (int)hi.y;
            }
            return o;
        }
    };
    auto load_b = [&](const uint8_t *W, int kc, int scol) -> Op {
        const uint8_t *colp = W + (kc * BN + scol) * 16;
        if constexpr (MF == 16) {
            const uint32_t d = *reinterpret_cast<const uint32_t *>(colp + 4 * g);
            return pack2(q40_lo(d), q40_hi(d));
        } else {
            const uint2 d = *reinterpret_cast<const uint2 *>(colp + 8 * g);
            Op o;
            o[0] = (int)q40_lo(d.x);
            o[1] = (int)q40_lo(d.y);
            o[2] = (int)q40_hi(d.x);
            o[3] = (int)q40_hi(d.y);
            return o;
        }
    };

    // One stage of arithmetic on the operands held in buffer A.
    auto compute_stage = [&](const uint8_t *A, int kb0, auto nact_tag) {
        constexpr int NA = decltype(nact_tag)::value; // row tiles with data
        auto active = [&](int i) { return i < NA; };
        const uint8_t *W = A + C::kLdsA;
        const float *Da = reinterpret_cast<const float *>(W + C::kLdsW);
        const float2 *Dw = reinterpret_cast<const float2 *>(W + C::kLdsW + C::kLdsDa);
        const int kvalid = B - kb0; // >= 1
        // eight-wave workgroups: wave priority 1 for the first half of the
        // wave's blocks of the stage, 0 for the second, so that the two waves
        // of a SIMD reach the stage barrier closer together (2-3% on the
        // 8-bit 64 x 160 shapes)
        if (C::kWaves >= 8)
            __builtin_amdgcn_s_setprio(1);

#pragma unroll
        for (int kk = 0; kk < KC / WK; kk++) {
            const int kc = kk * WK + wk;
            if (C::kWaves >= 8 && kk == (KC / WK) / 2)
                __builtin_amdgcn_s_setprio(0);
            if (kc >= kvalid)
                break;
            Op a[TM];
#pragma unroll
            for (int i = 0; i < TM; i++)
                if (active(i))
                    a[i] = load_a(A, kc, swz((wm * TM + i) * MF + rc, kc));

            if (MODE == kSums) {
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const Op b = load_b(W, kc, (wn * TN + j) * MF + rc);
                    const int64_t col = col0 + (wn * TN + j) * MF + rc;
#pragma unroll
                    for (int i = 0; i < TM; i++) {
                        const Acc D = M::mma(a[i], b, magic);
#pragma unroll
                        for (int r = 0; r < RG; r++) {
                            const int64_t row = row0 + (wm * TM + i) * MF + M::out_row(g, r);
                            if (row >= p.m0 && row < p.m1 && col >= p.n0 && col < p.n1)
                                p.sums[((row - p.m0) * (p.n1 - p.n0) + (col - p.n0)) * B + kb0 + kc] =
                                    (D[r] - kMagicBits) >> C::kShift;
                        }
                    }
                }
            } else {
                // row scales of the lane's result rows, four consecutive rows at a time
                float4 da[TM][RG / 4];
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int q = 0; q < RG / 4; q++)
                        if (active(i))
                            da[i][q] = *reinterpret_cast<const float4 *>(
                                Da + kc * BM + (wm * TM + i) * MF + M::out_row(g, 4 * q));
                // Software pipeline over the column tiles: the matrix
                // instructions of tile j are issued before the epilogue of
                // tile j-1, so their latency hides behind VALU work.  Padded
                // rows (past row_end) are computed too and never stored.
                Acc Dp[TM];
                float2 dwp = make_float2(0.0f, 0.0f);
#pragma unroll
                for (int j = 0; j <= TN; j++) {
                    Acc Dc[TM];
                    float2 dwc = make_float2(0.0f, 0.0f);
                    if (j < TN) {
                        const Op b = load_b(W, kc, (wn * TN + j) * MF + rc);
                        dwc = Dw[kc * BN + (wn * TN + j) * MF + rc];
#pragma unroll
                        for (int i = 0; i < TM; i++)
                            if (active(i))
                                Dc[i] = M::mma(a[i], b, magic);
                    }
                    if (j > 0) {
#pragma unroll
                        for (int i = 0; i < TM; i++) {
                            if (!active(i))
                                continue;
#pragma unroll
                            for (int q = 0; q < RG / 4; q++) {
                                const float dq[4] = {da[i][q].x, da[i][q].y, da[i][q].z, da[i][q].w};
#pragma unroll
                                for (int e = 0; e < 4; e++) {
                                    const int r = 4 * q + e;
                                    const float t = __builtin_fmaf(__int_as_float(Dp[i][r]), dwp.x, dwp.y);
                                    acc[i][j - 1][r] = __builtin_fmaf(t, dq[e], acc[i][j - 1][r]);
                                }
                            }
                        }
                    }
                    if (j < TN) {
#pragma unroll
                        for (int i = 0; i < TM; i++)
                            Dp[i] = Dc[i];
                        dwp = dwc;
                    }
                }
            }
        }
    };

    const int nstages = (B + KC - 1) / KC;
    if (KC <= B)
        load_stage(0, std::true_type{});
    else
        load_stage(0, std::false_type{});
    store_stage(lds);
    __syncthreads();

    // Stages alternate between the two buffers; the loop is unrolled by two
    // so that every LDS address carries its buffer offset as an immediate.
    for (int s = 0; s < nstages; s += 2) {
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const int st = s + half;
            if (st < nstages) {
                const int kb0 = st * KC;
                const bool more = st + 1 < nstages;
                if (more) {
                    if (kb0 + 2 * KC <= B)
                        load_stage(kb0 + KC, std::true_type{});
                    else
                        load_stage(kb0 + KC, std::false_type{});
                }
                if constexpr (MODE == kGrouped)
                    with_count<TM>(nact, [&](auto na) { compute_stage(lds + half * C::kStage, kb0, na); });
                else
                    compute_stage(lds + half * C::kStage, kb0, std::integral_constant<int, TM>{});
                if (more)
                    store_stage(lds + (half ^ 1) * C::kStage);
                __syncthreads();
            }
        }
    }

    if (MODE == kSums)
        return;

    // ---- fixed-order sum of the K-split partials of each wave group (wk = 0,
    //      1, ... in order); the waves of a group share the stores.  The
    //      widening factor 2^kShift is removed here.
    const float unscale = 1.0f / (float)(1 << C::kShift);
    float *red = reinterpret_cast<float *>(lds);
    constexpr int R = C::kRedTiles;
    for (int t0 = 0; t0 < C::kTiles; t0 += R) {
#pragma unroll
        for (int t = 0; t < C::kTiles; t++) {
            if (t < t0 || t >= t0 + R)
                continue;
            const int i = t / TN, j = t % TN;
#pragma unroll
            for (int r = 0; r < RG; r++)
                red[(((grp * WK + wk) * R + (t - t0)) * RG + r) * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();
        for (int tt = wk; tt < R && t0 + tt < C::kTiles; tt += WK) {
            const int t = t0 + tt;
            const int i = t / TN, j = t % TN;
            const int64_t col = col0 + (wn * TN + j) * MF + rc;
#pragma unroll
            for (int r = 0; r < RG; r++) {
                float v = red[(((grp * WK + 0) * R + tt) * RG + r) * 64 + lane];
#pragma unroll
                for (int w = 1; w < WK; w++)
                    v += red[(((grp * WK + w) * R + tt) * RG + r) * 64 + lane];
                const int rl = M::out_row(g, r);
                if (rl < vrows[i])
                    store_y(p, (row0 + (wm * TM + i) * MF + rl) * p.ldy + col, v * unscale);
            }
        }
        __syncthreads();
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

template <class C>
hipError_t launch_dense_cfg(const GemmProblem &p, hipStream_t stream)
{
    const int tm = (int)((p.rows + C::BM - 1) / C::BM), tn = (int)(p.n / C::BN);
    return launch_cfg<C, kGemm>(p, tm, tn, 0, 0, (int64_t)tm * tn, stream);
}

// Dense tile shapes.  The wide shapes run one 8-wave workgroup per CU whose
// waves advance together through the stage barriers (two independent
// workgroups on one CU finish at different times: the older one gets issue
// priority and the younger then runs alone).  KC = 8 blocks per stage.
template <int BITS> struct Tiles {
    // 64 x 160: two row halves of 32 x 160 (32x32 tiles), K split in four
    using W64x160 = Cfg<BITS, 32, 1, 5, 2, 1, 4, 8>;
    // 64 x 128: two row halves of 32 x 128, K split in four
    using W64x128 = Cfg<BITS, 32, 1, 4, 2, 1, 4, 8>;
    // 64 x 64 and 64 x 32: four waves of 16x16 tiles, K split in four (two
    // workgroups per CU)
    using T64x64 = Cfg<BITS, 16, 4, 4, 1, 1, 4, 8>;
    using T64x32 = Cfg<BITS, 16, 4, 2, 1, 1, 4, 8>;
    // small M: 16 rows, K split in four
    using T16x64 = Cfg<BITS, 16, 1, 4, 1, 1, 4, 8>;
    using T16x32 = Cfg<BITS, 16, 1, 2, 1, 1, 4, 8>;
};

constexpr int kCUs = 256;

// Estimated time of a shape: rounds of resident workgroups times the per-wave
// issue cost of one block (two VALU per result register, operand unpacking
// per row and column tile, matrix instruction issue per tile), times the
// waves that share a SIMD.
template <class C>
double est_cfg(int64_t m, int64_t n)
{
    if (n % C::BN != 0)
        return 1e300;
    const int64_t tiles = ((m + C::BM - 1) / C::BM) * (n / C::BN);
    const int64_t slots = (int64_t)C::kOcc * kCUs;
    const double rounds = (double)((tiles + slots - 1) / slots);
    const double wide = C::MF == 32 ? 2.0 : 1.0;
    const double cost = 2.0 * C::kRegs * C::kTiles + wide * (3.0 * C::TM + 5.0 * C::TN) +
                        2.0 * wide * C::kTiles;
    return rounds * cost * (C::kWaves * C::kOcc / 4.0);
}

// The kernel a dense problem runs (decided on the host from the shape alone,
// so the routing query below names exactly what launch_gemm launches).
template <int BITS>
int plan_dense_bits(const GemmProblem &p)
{
    using T = Tiles<BITS>;
    const int64_t m = p.rows, n = p.n;
    if (m <= 16)
        return est_cfg<typename T::T16x64>(m, n) <= est_cfg<typename T::T16x32>(m, n)
                   ? kTiled16x64
                   : kTiled16x32;
    const double e[4] = {est_cfg<typename T::W64x160>(m, n), est_cfg<typename T::W64x128>(m, n),
                         est_cfg<typename T::T64x64>(m, n), est_cfg<typename T::T64x32>(m, n)};
    int best = 3;
    for (int i = 0; i < 3; i++)
        if (e[i] < e[best])
            best = i;
    // 4-bit activations run the direct-load kernels: 64 x 160 tiles where
    // they are the estimate's choice (wide.hip), else 32 x 128 strips
    // (strip.hip), which measured as fast as or faster than the 64 x 128,
    // 64 x 64 and 64 x 32 tiles on every shape tried (K = 2048 .. 5120,
    // M = 128 .. 4096, N = 1536 .. 17408: up to 18% faster).  8-bit codes
    // run the strip kernel too (up to 33% faster than the tiled kernel),
    // except where the estimate picks 64 x 160 tiles and there are fewer
    // strips than three per CU: there the tiled kernel's K-split workgroups
    // fill every CU and the strips do not (M = 512, K = 17408, N = 5120).
    if (BITS == 4 && best == 0 && wide_fits(p))
        return kWide;
    if (strip_fits(p) &&
        (BITS == 4 || best != 0 || (p.rows + 31) / 32 * (p.n / 128) >= 3 * kCUs))
        return kStrip;
    static const int tiled[4] = {kTiled64x160, kTiled64x128, kTiled64x64, kTiled64x32};
    return tiled[best];
}

template <int BITS>
hipError_t launch_dense_bits(int kernel, const GemmProblem &p, hipStream_t stream)
{
    using T = Tiles<BITS>;
    switch (kernel) {
    case kWide: return launch_wide(p, stream);
    case kStrip: return launch_strip(p, stream);
    case kTiled64x160: return launch_dense_cfg<typename T::W64x160>(p, stream);
    case kTiled64x128: return launch_dense_cfg<typename T::W64x128>(p, stream);
    case kTiled64x64: return launch_dense_cfg<typename T::T64x64>(p, stream);
    case kTiled64x32: return launch_dense_cfg<typename T::T64x32>(p, stream);
    case kTiled16x64: return launch_dense_cfg<typename T::T16x64>(p, stream);
    default: return launch_dense_cfg<typename T::T16x32>(p, stream);
    }
}

// Grouped: 32-row slots (row tiles past an expert's rows are skipped) and
// 128, 64 or 32 columns per workgroup: four waves of 32 x 32, each over the
// whole of K (an expert's K is short, so splitting it across waves would leave
// each wave too few blocks to amortise its set-up and the final reduction).
template <int BITS> struct GroupedTiles {
    using C128 = Cfg<BITS, 16, 2, 2, 1, 4, 1, 4>; // 32 x 128
    using C64 = Cfg<BITS, 16, 2, 2, 1, 2, 1, 4>;  // 32 x 64
    using C32 = Cfg<BITS, 16, 2, 2, 1, 1, 1, 4>;  // 32 x 32
};

template <class C>
hipError_t launch_grouped_cfg(const GemmProblem &p, hipStream_t stream)
{
    // every expert needs ceil(rows_e / BM) slots: bounded by both of these
    int64_t slots = (p.rows + p.experts * (C::BM - 1)) / C::BM;
    if (slots > p.rows)
        slots = p.rows;
    const int tn = (int)(p.n / C::BN);
    return launch_cfg<C, kGrouped>(p, 0, tn, 0, 0, slots * tn, stream);
}

template <int BITS>
hipError_t launch_grouped_bits(int kernel, const GemmProblem &p, hipStream_t stream)
{
    using T = GroupedTiles<BITS>;
    switch (kernel) {
    case kGrouped128: return launch_grouped_cfg<typename T::C128>(p, stream);
    case kGrouped64: return launch_grouped_cfg<typename T::C64>(p, stream);
    default: return launch_grouped_cfg<typename T::C32>(p, stream);
    }
}

template <int BITS>
hipError_t launch_sums_bits(const GemmProblem &p, hipStream_t stream)
{
    // the 32x32 main loop of the wide dense shapes, one 32x32 tile per workgroup
    using C = Cfg<BITS, 32, 1, 1, 1, 1, 4, 8>;
    const int tm0 = (int)(p.m0 / C::BM), tm1 = (int)((p.m1 + C::BM - 1) / C::BM);
    const int tn0 = (int)(p.n0 / C::BN), tn1 = (int)((p.n1 + C::BN - 1) / C::BN);
    const int tm = tm1 - tm0, tn = tn1 - tn0;
    return launch_cfg<C, kSums>(p, tm, tn, tm0, tn0, (int64_t)tm * tn, stream);
}

} // namespace

int plan_gemm(const GemmProblem &p)
{
    if (p.rows == 0)
        return kNoKernel;
    if (skinny_fits(p))
        return kSkinny;
    return p.act_bits == 4 ? plan_dense_bits<4>(p) : plan_dense_bits<8>(p);
}

int plan_grouped_gemm(const GemmProblem &p)
{
    if (p.rows == 0)
        return kNoKernel;
    if (grouped_wide_fits(p))
        return kSlot;
    return p.n % 128 == 0 ? kGrouped128 : p.n % 64 == 0 ? kGrouped64 : kGrouped32;
}

const char *kernel_name(int kernel)
{
    switch (kernel) {
    case kSkinny: return "weight-stream";
    case kWide: return "wide 64x160";
    case kStrip: return "strip 32x128";
    case kTiled64x160: return "tiled 64x160";
    case kTiled64x128: return "tiled 64x128";
    case kTiled64x64: return "tiled 64x64";
    case kTiled64x32: return "tiled 64x32";
    case kTiled16x64: return "tiled 16x64";
    case kTiled16x32: return "tiled 16x32";
    case kSlot: return "expert-slot";
    case kGrouped128: return "grouped 32x128";
    case kGrouped64: return "grouped 32x64";
    case kGrouped32: return "grouped 32x32";
    default: return "none";
    }
}

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream)
{
    const int kernel = plan_gemm(p);
    if (kernel == kNoKernel)
        return hipSuccess;
    if (kernel == kSkinny)
        return launch_skinny(p, stream);
    return p.act_bits == 4 ? launch_dense_bits<4>(kernel, p, stream)
                           : launch_dense_bits<8>(kernel, p, stream);
}

hipError_t launch_grouped_gemm(const GemmProblem &p, hipStream_t stream)
{
    const int kernel = plan_grouped_gemm(p);
    if (kernel == kNoKernel)
        return hipSuccess;
    if (kernel == kSlot)
        return launch_grouped_wide(p, stream);
    return p.act_bits == 4 ? launch_grouped_bits<4>(kernel, p, stream)
                           : launch_grouped_bits<8>(kernel, p, stream);
}

hipError_t launch_blocksums(const GemmProblem &p, hipStream_t stream)
{
    if (p.m1 <= p.m0 || p.n1 <= p.n0)
        return hipSuccess;
    return p.act_bits == 4 ? launch_sums_bits<4>(p, stream) : launch_sums_bits<8>(p, stream);
}

} // namespace bpg
