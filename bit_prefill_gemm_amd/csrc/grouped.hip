// grouped.hip -- the grouped (expert) W4A4 product on 64-row expert slots
// (gfx950, 4-bit activations).
//
// "Where the engine is going: HRX and the NPU", section "4-bit activations
// reach the MoE experts": the rotated 4-bit route also runs the expert
// matmuls, every expert multiplying its own rows by its own weights.  With a
// few dozen rows per expert each expert's weights are streamed once, and the
// arithmetic is the epilogue-bound block product of the dense wide kernel
// (wide.hip), whose operand layout this kernel keeps: image blocks copied
// verbatim into LDS by direct loads, activation rows with their 16-byte
// blocks XOR-swizzled by row, row scales stored [block][row],
// v_mfma_i32_32x32x32_i8 per 32x32 tile and block with the next tile's
// instruction issued before the previous tile's epilogue.  On top:
//   - 64-row expert slots: an expert with r rows owns ceil(r / 64) slots, and
//     a work item is one slot and 128 columns (four 32-column tiles).  Each
//     of the workgroup's four waves owns one tile over the whole of K (no
//     partial sums to add across waves); it computes the item's rows 0..31,
//     and rows 32..63 in a second pass only when the item has them, so no
//     arithmetic goes to an empty 32-row half;
//   - a persistent grid of two workgroups per CU, each walking its items
//     (every G-th one) and their stages of eight blocks as one double-
//     buffered pipeline across item boundaries; the two workgroups of a CU
//     run independently, so one computes while the other waits for its
//     loads at its barrier;
//   - a slot table built once per workgroup in LDS from the device-side
//     expert offsets (clamped row starts, inclusive ends of the slots with
//     more and with at most 32 rows); an item finds its expert with one LDS
//     read and four ballots per 256 experts.  Items are numbered slots with
//     more than 32 rows first, so that the round-robin split gives every
//     workgroup nearly the same work;
//   - rows read through an optional row index (the gathered product), looked
//     up one item ahead so that the index loads are in flight during the
//     current item's stages.
// Every output is one wave's in-order accumulation over the blocks of K (no
// partial sums are added across waves), so the result is bit-identical from
// run to run and to the same product on explicitly permuted rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "operands.h"

namespace bpg {

namespace {

constexpr int kMaxTableExperts = 1024;

struct GroupedCfg {
    static constexpr int TN = 4;                     // 32-column tiles per item, one per wave
    static constexpr int BM = 64, BN = 32 * TN;
    static constexpr int kThreads = 256;             // 4 waves; two workgroups per CU
    static constexpr int kGroupBytes = 2304;         // image block: 32 columns x 4 K-blocks
    static constexpr int kSB = 8;                    // blocks per stage (two groups)
    static constexpr int kWTile = 2 * kGroupBytes;   // one tile's two groups of a stage
    // one stage in LDS: image blocks [tile][group] verbatim, codes [row][8
    // blocks] (16-byte blocks XOR-swizzled by row), row scales [block][row]
    static constexpr int kW = TN * kWTile;
    static constexpr int kA = BM * kSB * 16;
    static constexpr int kDa = kSB * BM * 4;
    static constexpr int kBuf = kW + kA + kDa;
    static_assert(kW == 16 * 1024 + 8 * 256, "weights: 16 wave-wide 16-byte loads + 8 4-byte ones");
    static_assert(2 * (2 * kBuf + 12 * (kMaxTableExperts + 2) + 2 * 256) <= 160 * 1024,
                  "LDS budget of two workgroups per CU");
};

// One work item: its row range, expert and column tile (uniform), and this
// lane's direct-load offsets: code chunks of rows 8 (wave + 4u) + lane / 8
// (u = 0, 1) and the row scale of row `lane`.
struct Item {
    int row0;
    int rows;      // 1 .. 64 rows of the slot that hold data
    int expert;
    int ct;        // 128-column tile
    uint32_t aoff[2], daoff;
};

__global__ __launch_bounds__(256, 2) void grouped_kernel(GemmProblem p, int tiles_n)
{
    typedef GroupedCfg C;
    typedef Mfma<32> M;
    typedef M::Op Op;
    typedef M::Acc Acc;
    // two stage buffers, each its own array (the compiler tells the direct
    // loads into one from the reads of the other by the array they address)
    __shared__ __attribute__((aligned(16))) uint8_t buf0[C::kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[C::kBuf];
    // slot table: clamped row start of expert e (e <= experts), and the
    // inclusive ends of its slots with more than 32 rows (full_end[e] = such
    // slots of experts 0..e) and of its slots with at most 32 (half_end)
    __shared__ __attribute__((aligned(16))) int row_start[kMaxTableExperts + 4];
    __shared__ __attribute__((aligned(16))) int full_end[kMaxTableExperts];
    __shared__ __attribute__((aligned(16))) int half_end[kMaxTableExperts];
    // gathered source rows of an item's 64 rows, two items ahead
    __shared__ __attribute__((aligned(16))) int ids0[64];
    __shared__ __attribute__((aligned(16))) int ids1[64];
    __shared__ int wave_sum[2][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;  // operand row / column, result column
    const int hk = lane >> 5; // operand K half, result row group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // = the wave's tile

    const int B = (int)(p.k / 32); // the host limits K to 2^22
    const int NG = (B + 3) / 4;
    const int nst = (NG + 1) / 2;  // stages of two groups
    const int64_t arow = p.k / 2;
    const int64_t ntiles32 = p.n / 32;
    const int E = (int)p.experts;  // <= kMaxTableExperts
    const int rows_all = (int)p.rows;
    const bool gather = p.row_ids != nullptr;

    // ---- slot table.  Thread t counts the slots of experts 4t .. 4t+3: an
    //      expert with r rows has r / 64 slots of 64 rows and, when r % 64 is
    //      not zero, one of r % 64 rows; a slot is full when it has more
    //      than 32 rows (it then takes a second pass).
    for (int e = tid; e <= kMaxTableExperts; e += C::kThreads) {
        int r = rows_all;
        if (e <= E) {
            const int o = p.offsets[e];
            r = o < 0 ? 0 : (o > rows_all ? rows_all : o);
        }
        row_start[e] = r;
    }
    __syncthreads();
    int nf[4], nh[4], own_f = 0, own_h = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int e = 4 * tid + u;
        nf[u] = nh[u] = 0;
        if (e < E) {
            const int a = row_start[e], b = row_start[e + 1];
            const int r = b > a ? b - a : 0;
            nf[u] = r / C::BM + (r % C::BM > 32 ? 1 : 0);
            nh[u] = (r % C::BM != 0 && r % C::BM <= 32) ? 1 : 0;
        }
        own_f += nf[u];
        own_h += nh[u];
    }
    int incl_f = own_f, incl_h = own_h; // inclusive scans over the workgroup
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int vf = __shfl_up(incl_f, d);
        const int vh = __shfl_up(incl_h, d);
        if (lane >= d) {
            incl_f += vf;
            incl_h += vh;
        }
    }
    if (lane == 63) {
        wave_sum[0][wave] = incl_f;
        wave_sum[1][wave] = incl_h;
    }
    __syncthreads();
    for (int w = 0; w < wave; w++) {
        incl_f += wave_sum[0][w];
        incl_h += wave_sum[1][w];
    }
    {
        int run_f = incl_f - own_f, run_h = incl_h - own_h;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            run_f += nf[u];
            run_h += nh[u];
            full_end[4 * tid + u] = run_f;
            half_end[4 * tid + u] = run_h;
        }
    }
    const int full_slots = wave_sum[0][0] + wave_sum[0][1] + wave_sum[0][2] + wave_sum[0][3];
    const int half_slots = wave_sum[1][0] + wave_sum[1][1] + wave_sum[1][2] + wave_sum[1][3];
    const int total_slots = full_slots + half_slots;
    __syncthreads();

    const int64_t items = (int64_t)total_slots * tiles_n;
    const int G = (int)gridDim.x;
    const int L = xcd_remap(blockIdx.x, G);
    const int nmine = L < items ? (int)((items - L + G - 1) / G) : 0;
    if (nmine == 0)
        return; // uniform across the workgroup
    const int nchunks = (E + 255) / 256;

    // ---- item k of this workgroup: expert, row range, column tile.  Items
    //      are numbered full slots first, then the others (slot-major, 128-
    //      column tiles minor), and workgroup L takes items L, L + G, ...: so
    //      every workgroup gets nearly the same number of each kind.
    auto locate = [&](Item &it, int k) __attribute__((always_inline)) {
        int idx = L + G * k; // < items < 2^31
        const bool is_full = idx < full_slots * tiles_n;
        if (!is_full)
            idx -= full_slots * tiles_n;
        const int s = idx / tiles_n;
        it.ct = idx - s * tiles_n;
        const int *ends = is_full ? full_end : half_end;
        int e = 0;
        for (int ch = 0; ch < nchunks; ch++) {
            const int4 v = *reinterpret_cast<const int4 *>(&ends[256 * ch + 4 * lane]);
            e += __popcll(__ballot(v.x <= s)) + __popcll(__ballot(v.y <= s)) +
                 __popcll(__ballot(v.z <= s)) + __popcll(__ballot(v.w <= s));
        }
        e = __builtin_amdgcn_readfirstlane(e);
        const int first = __builtin_amdgcn_readfirstlane(e > 0 ? ends[e - 1] : 0);
        const int rs = __builtin_amdgcn_readfirstlane(row_start[e]);
        const int re = __builtin_amdgcn_readfirstlane(row_start[e + 1]);
        // a full slot j is the expert's slot j; the short one is its last
        it.row0 = rs + C::BM * (is_full ? s - first : (re - rs) / C::BM);
        it.rows = re - it.row0 < C::BM ? re - it.row0 : C::BM;
        it.expert = e;
    };
    // When gathering, the source rows of item k's 64 rows (rows past its
    // rows repeat its last row) are copied into an LDS slot by wave 0 with one
    // direct load, two items before they are needed.
    auto fetch_ids = [&](int *slot, int k) __attribute__((always_inline)) {
        Item it;
        locate(it, k);
        const int rr = lane < it.rows - 1 ? lane : it.rows - 1;
        const uint8_t *src = uniform(reinterpret_cast<const uint8_t *>(p.row_ids + it.row0));
        __builtin_amdgcn_global_load_lds((glb_void *)(src + opaque((uint32_t)(4 * rr))),
                                         (lds_void *)slot, 4, 0, 0);
    };
    // item k with this lane's load offsets (ids: its slot of source rows)
    auto make_item = [&](Item &it, int k, const int *ids) __attribute__((always_inline)) {
        locate(it, k);
        const int last = it.rows - 1;
        int32_t src[3];
#pragma unroll
        for (int u = 0; u < 3; u++) {
            const int row = u < 2 ? 8 * (wave + 4 * u) + (lane >> 3) : lane;
            const int rr = row < last ? row : last;
            int32_t r = rr;
            if (gather) {
                r = ids[rr];
                r = r < 0 ? 0 : (r >= p.src_rows ? (int32_t)(p.src_rows - 1) : r);
            }
            src[u] = r;
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int row = 8 * (wave + 4 * u) + (lane >> 3);
            const int ablk = (lane & 7) ^ (row & 7);
            it.aoff[u] = (uint32_t)(src[u] * arow + ablk * 16);
        }
        it.daoff = (uint32_t)((int64_t)src[2] * B * 4);
    };

    // weights: byte b of a stage's copy (b = 1024 (wave + 4u) + 16 lane for
    // the 16-byte loads u < 4, 16384 + 256 (wave + 4u') + 4 lane for the
    // 4-byte loads u' < 2) is byte b % 2304 of group 2 st + gg of tile t
    uint32_t woff[6];
    uint32_t wgg = 0; // bit u: the load's group within the stage
#pragma unroll
    for (int u = 0; u < 6; u++) {
        const int b = u < 4 ? 1024 * (wave + 4 * u) + 16 * lane
                            : 16384 + 256 * (wave + 4 * (u - 4)) + 4 * lane;
        const int t = b / C::kWTile;
        const int r = b % C::kWTile;
        const int gg = r / C::kGroupBytes;
        woff[u] = (uint32_t)((t * NG + gg) * C::kGroupBytes + r % C::kGroupBytes);
        wgg |= (uint32_t)gg << u;
    }

    // Stage st of an item into a buffer.  A stage inside K takes fixed lane
    // offsets from uniform bases.  In the last stage, code chunks of blocks
    // past K are written as zeros instead of loaded: a zero code makes the
    // block's product exactly zero whatever the weights (a group past the
    // image repeats group NG-1, scales repeat block B-1), so the arithmetic
    // always runs over all eight blocks.  An item of at most 32 rows loads no
    // code rows past 32 (never read).
    auto issue = [&](const Item &it, uint8_t *buf, int st) __attribute__((always_inline)) {
        const int g0 = 2 * st;
        const uint8_t *wst = uniform(
            p.wcodes + (((int64_t)it.expert * ntiles32 + 4 * it.ct) * NG + g0) * C::kGroupBytes);
        const uint8_t *ast =
            uniform(p.codes + (gather ? 0 : (int64_t)it.row0 * arow) + (size_t)st * (C::kSB * 16));
        const uint8_t *dst = uniform(reinterpret_cast<const uint8_t *>(
            p.scales + (gather ? 0 : (int64_t)it.row0 * B) + C::kSB * st));
        uint8_t *wl = buf;
        uint8_t *al = buf + C::kW;
        uint8_t *dl = buf + C::kW + C::kA;
        const bool tail = C::kSB * (st + 1) > B;
        const bool over_g = g0 + 1 >= NG; // the stage's second group is past the image
#pragma unroll
        for (int u = 0; u < 6; u++) {
            const uint32_t o =
                woff[u] - (tail && over_g && ((wgg >> u) & 1) ? (uint32_t)C::kGroupBytes : 0u);
            if (u < 4)
                __builtin_amdgcn_global_load_lds((glb_void *)(wst + opaque(o)),
                                                 (lds_void *)(wl + 1024 * (wave + 4 * u)), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((glb_void *)(wst + opaque(o)),
                                                 (lds_void *)(wl + 16384 + 256 * (wave + 4 * (u - 4))),
                                                 4, 0, 0);
        }
        const int nu = it.rows > 32 ? 2 : 1;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            if (u < nu) {
                uint8_t *dstl = al + 1024 * (wave + 4 * u);
                const int row = 8 * (wave + 4 * u) + (lane >> 3);
                if (!tail || C::kSB * st + ((lane & 7) ^ (row & 7)) < B)
                    __builtin_amdgcn_global_load_lds((glb_void *)(ast + opaque(it.aoff[u])),
                                                     (lds_void *)dstl, 16, 0, 0);
                else
                    *reinterpret_cast<uint4 *>(dstl + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int i = wave + 4 * u; // block of the stage, lane = row
            const int blk = C::kSB * st + i < B ? i : B - 1 - C::kSB * st;
            __builtin_amdgcn_global_load_lds((glb_void *)(dst + opaque(it.daoff + 4 * blk)),
                                             (lds_void *)(dl + 256 * i), 4, 0, 0);
        }
    };

    // partial sums of the wave's tile for rows 0..31 and 32..63
    float acc_lo[16], acc_hi[16];
#pragma unroll
    for (int r = 0; r < 16; r++)
        acc_lo[r] = acc_hi[r] = 0.0f;
    Acc magic;
#pragma unroll
    for (int r = 0; r < 16; r++)
        magic[r] = kMagicBits;

    // LDS read offsets inside a buffer (each read address is its array plus
    // one integer offset: longer address chains lose the array's identity,
    // and the compiler then waits for the direct loads into the other buffer
    // before the read).  Weight slots 2hk, 2hk+1 of the lane's column and its
    // fp16 scales in group g of the wave's tile (+ 2304 g); codes of row c,
    // bytes 8hk..8hk+7 (block q at slot q ^ (c & 7)); row scales of the
    // lane's result rows 4hk + 8 r4 .. + 3 of block q (+ 256 q).  Rows 32..63
    // add 4096 bytes of codes and 128 of scales.
    const uint32_t w_rd = opaque((uint32_t)(wave * C::kWTile + ((2 * hk) * 32 + c) * 16));
    const uint32_t hw_rd =
        opaque((uint32_t)(wave * C::kWTile + 2048 + ((c & 15) * 2 + (c >> 4)) * 8));
    const uint32_t a_rd = opaque((uint32_t)(C::kW + c * 128 + 8 * hk));
    const uint32_t d_rd = opaque((uint32_t)(C::kW + C::kA + 4 * hk * 4));
    const int csw = c & 7;

    // 32 rows (byte offsets ah, dh: rows 0..31 or 32..63) of the wave's tile
    // over the stage's eight blocks; the matrix instruction of block q+1 is
    // issued before the epilogue of block q.  Result register r of a lane
    // holds row 8 (r / 4) + 4 hk + r % 4: with ng = 1 (compiled in) only the
    // first 8-row group gets an epilogue, for a second pass whose rows all
    // lie in it (the common case: an expert slot of 33..40 rows).
    auto compute = [&](auto ng_tag, float (&acc)[16], const uint8_t *buf, uint32_t ah,
                       uint32_t dh) __attribute__((always_inline)) {
        constexpr int ng = decltype(ng_tag)::value;
        uint4 wr[2][2];
        uint2 hw[2];
#pragma unroll
        for (int g = 0; g < 2; g++) {
            wr[g][0] = *reinterpret_cast<const uint4 *>(buf + (w_rd + g * C::kGroupBytes));
            wr[g][1] = *reinterpret_cast<const uint4 *>(buf + (w_rd + g * C::kGroupBytes + 512));
            hw[g] = *reinterpret_cast<const uint2 *>(buf + (hw_rd + g * C::kGroupBytes));
        }
        Acc Dp;
        float dwp = 0.0f, nbp = 0.0f;
        float4 dap[4];
        // the activation operand of block q is read one block ahead, so its
        // LDS latency overlaps block q-1's matrix instruction and epilogue
        uint2 adn = *reinterpret_cast<const uint2 *>(buf + (ah + a_rd + (uint32_t)(csw * 16)));
#pragma unroll
        for (int q = 0; q <= C::kSB; q++) {
            Acc Dc;
            float dwc = 0.0f, nbc = 0.0f;
            float4 dac[4];
            if (q < C::kSB) {
                const uint2 ad = adn;
                if (q + 1 < C::kSB)
                    adn = *reinterpret_cast<const uint2 *>(
                        buf + (ah + a_rd + (uint32_t)(((q + 1) ^ csw) * 16)));
                Op a;
                a[0] = (int)act_lo(ad.x);
                a[1] = (int)act_lo(ad.y);
                a[2] = (int)act_hi(ad.x);
                a[3] = (int)act_hi(ad.y);
#pragma unroll
                for (int r4 = 0; r4 < ng; r4++)
                    dac[r4] = *reinterpret_cast<const float4 *>(
                        buf + (dh + d_rd + q * 256 + r4 * 32));
                const int g = q >> 2, qq = q & 3;
                const uint32_t x = qq == 0 ? wr[g][0].x : qq == 1 ? wr[g][0].y : qq == 2 ? wr[g][0].z : wr[g][0].w;
                const uint32_t y = qq == 0 ? wr[g][1].x : qq == 1 ? wr[g][1].y : qq == 2 ? wr[g][1].z : wr[g][1].w;
                Op bo;
                bo[0] = (int)q40_lo(x);
                bo[1] = (int)q40_lo(y);
                bo[2] = (int)q40_hi(x);
                bo[3] = (int)q40_hi(y);
                Dc = M::mma(a, bo, magic);
                const uint32_t hd = qq < 2 ? hw[g].x : hw[g].y;
                // converted here, so that the epilogue is plain fp32 FMAs
                dwc = __uint_as_float(opaque(__float_as_uint(
                    half_bits_to_float((uint16_t)((qq & 1) ? hd >> 16 : hd & 0xFFFFu)))));
                nbc = -kMagic * dwc;
            }
            if (q > 0) {
#pragma unroll
                for (int r4 = 0; r4 < ng; r4++) {
                    const float dq[4] = {dap[r4].x, dap[r4].y, dap[r4].z, dap[r4].w};
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int r = 4 * r4 + e;
                        const float t = __builtin_fmaf(__int_as_float(Dp[r]), dwp, nbp);
                        acc[r] = __builtin_fmaf(t, dq[e], acc[r]);
                    }
                }
            }
            Dp = Dc;
            dwp = dwc;
            nbp = nbc;
#pragma unroll
            for (int r4 = 0; r4 < ng; r4++)
                dap[r4] = dac[r4];
            // one block at a time: hoisting later blocks' matrix instructions
            // above these epilogues keeps all their results live at once
            __builtin_amdgcn_sched_barrier(0);
        }
        // the epilogues finish here: sunk past a following pass they would
        // keep this pass's matrix results live through it
#pragma unroll
        for (int r = 0; r < 16; r++)
            asm volatile("" : "+v"(acc[r]));
    };

    // the wave's 32x32 tile of 32 rows (rbase: 0 or 32) of an item; the
    // widening factor 256 is removed here; acc is cleared
    auto store = [&](float (&acc)[16], const Item &it, int rbase) __attribute__((always_inline)) {
        const int64_t y0 = ((int64_t)it.row0 + rbase + 4 * hk) * p.ldy +
                           ((int64_t)it.ct * C::BN + wave * 32 + c);
        const int lim = it.rows - rbase - 4 * hk;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int ro = 8 * (r >> 2) + (r & 3);
            if (ro < lim)
                store_y(p, y0 + (int64_t)ro * p.ldy, acc[r] * (1.0f / 256.0f));
            acc[r] = 0.0f;
        }
    };

    // ---- the pipeline: pair (item, stage) s computes from buffer s % 2
    //      while pair s + 1 loads into the other.  Issue cursor: item ki,
    //      stage sti (icur); compute cursor: item kc, stage stc (ccur).
    Item icur, ccur;
    int ki = 0, sti = 0;
    if (gather) {
        if (wave == 0) {
            fetch_ids(ids0, 0);
            if (nmine > 1)
                fetch_ids(ids1, 1);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0)
        __syncthreads();
    }
    make_item(icur, 0, ids0);
    ccur = icur;
    issue(icur, buf0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    int kc = 0, stc = 0;
    auto step = [&](uint8_t *bc, uint8_t *bn) __attribute__((always_inline)) {
        if (sti + 1 < nst) {
            sti++;
            issue(icur, bn, sti);
        } else if (ki + 1 < nmine) {
            ki++;
            sti = 0;
            make_item(icur, ki, (ki & 1) ? ids1 : ids0);
            issue(icur, bn, 0);
        }
        // the source rows of item kc + 2 replace those of item kc
        if (gather && stc == 0 && wave == 0 && kc + 2 < nmine)
            fetch_ids((kc & 1) ? ids1 : ids0, kc + 2);
        typedef std::integral_constant<int, 1> OneGroup;
        typedef std::integral_constant<int, 4> AllGroups;
        compute(AllGroups{}, acc_lo, bc, 0u, 0u);
        if (ccur.rows > 40)
            compute(AllGroups{}, acc_hi, bc, 32u * 128u, 32u * 4u);
        else if (ccur.rows > 32)
            compute(OneGroup{}, acc_hi, bc, 32u * 128u, 32u * 4u);
        __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): the next pair has landed
        __syncthreads();
        if (++stc < nst)
            return false;
        store(acc_lo, ccur, 0);
        if (ccur.rows > 32)
            store(acc_hi, ccur, 32);
        if (++kc >= nmine)
            return true;
        stc = 0;
        locate(ccur, kc);
        return false;
    };
    for (;;) {
        if (step(buf0, buf1))
            break;
        if (step(buf1, buf0))
            break;
    }
}

} // namespace

bool grouped_wide_fits(const GemmProblem &p)
{
    if (p.act_bits != 4 || p.n % GroupedCfg::BN != 0 || p.experts < 1 ||
        p.experts > kMaxTableExperts || p.rows <= 0 || p.rows >= ((int64_t)1 << 31))
        return false;
    // gathered rows are addressed from row 0 with 32-bit lane offsets
    if (p.row_ids && (p.src_rows * (p.k / 2) >= ((int64_t)1 << 31) ||
                      p.src_rows * (p.k / 32) * 4 >= ((int64_t)1 << 31)))
        return false;
    // item indices stay below 2^31
    const int64_t slots = p.rows / GroupedCfg::BM + p.experts;
    return slots * (p.n / GroupedCfg::BN) < ((int64_t)1 << 31);
}

hipError_t launch_grouped_wide(const GemmProblem &p, hipStream_t stream)
{
    constexpr int kSlots = 2 * 256; // two workgroups on each of the 256 CUs
    const int64_t tiles_n = p.n / GroupedCfg::BN;
    // every expert needs ceil(rows_e / 64) slots: at most this many items
    int64_t slots = (p.rows + p.experts * (GroupedCfg::BM - 1)) / GroupedCfg::BM;
    if (slots > p.rows)
        slots = p.rows;
    const int64_t items = slots * tiles_n;
    const int grid = (int)(items < kSlots ? items : kSlots);
    if (grid <= 0)
        return hipSuccess;
    grouped_kernel<<<dim3((unsigned)grid), GroupedCfg::kThreads, 0, stream>>>(p, (int)tiles_n);
    return hipGetLastError();
}

} // namespace bpg
