// moe.hip -- the glue of an expert layer around the grouped product (gfx950):
// the expert sort of the routed rows and the weighted combine.
//
// "Where the engine is going: HRX and the NPU", section "4-bit activations
// reach the MoE experts": the route covers the expert matmuls.  The pages give
// no detail of the layer around them; this library's reading: every token t
// has topk routed choices (entry t*topk + j, expert e, weight w); the entries
// are sorted by expert, stably (entry order inside an expert), so that each
// expert's rows are contiguous for the grouped product, and the outputs of a
// token's choices are added in choice order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace bpg {

namespace {

constexpr int kSortThreads = 256;

// Inclusive scans of two ints per thread over the workgroup (kSortThreads),
// in thread order, with one pair of barriers; `wsum` is LDS of 2 *
// kSortThreads / 64 ints.
__device__ __forceinline__ int2 block_scan_incl2(int a, int b, int *wsum)
{
    constexpr int kW = kSortThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ia = a, ib = b;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int ua = __shfl_up(ia, d), ub = __shfl_up(ib, d);
        if (lane >= d) {
            ia += ua;
            ib += ub;
        }
    }
    if (lane == 63) {
        wsum[wave] = ia;
        wsum[kW + wave] = ib;
    }
    __syncthreads();
    int ba = 0, bb = 0;
    for (int w = 0; w < wave; w++) {
        ba += wsum[w];
        bb += wsum[kW + w];
    }
    __syncthreads();
    return make_int2(ba + ia, bb + ib);
}

// Counting sort with one workgroup per expert x.  Thread t owns the
// contiguous entry range [t*per, (t+1)*per) and counts its entries of experts
// before x and of x itself; the sum of the first counts over the workgroup is
// x's offset, and a scan of the second over the threads in order gives each
// entry of x its place: the stable order.  Expert ids outside [0, experts)
// are clamped (the rows stay in bounds).  Ranges of up to kCached entries
// read with 16-byte loads stay in registers between the count and the
// placement; longer ones are read again.
constexpr int kCached = 16;

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const int32_t *__restrict__ expert_of, int n, int topk, int experts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ row_token, int32_t *__restrict__ slot_of)
{
    __shared__ int wsum[2 * kSortThreads / 64];
    const int x = blockIdx.x, tid = threadIdx.x;
    const int per = (n + kSortThreads - 1) / kSortThreads;
    const int lo = tid * per < n ? tid * per : n;
    const int hi = lo + per < n ? lo + per : n;
    auto clamp_e = [&](int e) { return e < 0 ? 0 : (e >= experts ? experts - 1 : e); };
    auto expert_at = [&](int i) { return clamp_e(expert_of[i]); };
    // 16-byte loads where the range and the pointer allow them
    const bool vec = per % 4 == 0 && (reinterpret_cast<uintptr_t>(expert_of) & 15) == 0;
    const bool cached = vec && per <= kCached;
    int before = 0, mine = 0; // entries of experts below x, and of x
    auto count = [&](int e) {
        before += e < x;
        mine += e == x;
    };
    int ec[kCached]; // the range's experts when cached (entries past hi: -1)
    if (cached) {
#pragma unroll
        for (int u = 0; u < kCached / 4; u++) {
            const int i0 = lo + 4 * u;
            int ev[4] = {-1, -1, -1, -1};
            if (i0 + 4 <= hi) {
                const int4 v = *reinterpret_cast<const int4 *>(expert_of + i0);
                ev[0] = clamp_e(v.x);
                ev[1] = clamp_e(v.y);
                ev[2] = clamp_e(v.z);
                ev[3] = clamp_e(v.w);
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (i0 + j < hi)
                        ev[j] = expert_at(i0 + j);
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                ec[4 * u + j] = ev[j];
                if (ev[j] >= 0)
                    count(ev[j]);
            }
        }
    } else if (vec) {
        for (int i = lo; i + 4 <= hi; i += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(expert_of + i);
            const int ev[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; j++)
                count(clamp_e(ev[j]));
        }
        for (int i = lo + (hi - lo) / 4 * 4; i < hi; i++)
            count(expert_at(i));
    } else {
        for (int i = lo; i < hi; i++)
            count(expert_at(i));
    }
    // x's offset (the entries of the experts before it) and the places of
    // this thread's entries of x
    const int2 incl = block_scan_incl2(before, mine, wsum);
    int base_x = 0;
#pragma unroll
    for (int w = 0; w < kSortThreads / 64; w++)
        base_x += wsum[w];
    if (tid == 0) {
        offsets[x] = base_x;
        if (x == experts - 1)
            offsets[experts] = n; // every entry's (clamped) expert is at most x
    }
    if (mine == 0)
        return;
    int pos = base_x + incl.y - mine;
    if (cached) {
#pragma unroll
        for (int j = 0; j < kCached; j++)
            if (ec[j] == x) {
                slot_of[lo + j] = pos;
                row_token[pos] = (lo + j) / topk;
                pos++;
            }
        return;
    }
    for (int i = lo; i < hi; i++)
        if (expert_at(i) == x) {
            slot_of[i] = pos;
            row_token[pos] = i / topk;
            pos++;
        }
}

// y[t][c..c+3] = sum_j w[t k + j] * dn[slot[t k + j]][c..c+3], j ascending,
// every step one fp32 fma from 0.  One thread per 4 columns of a token.
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ dn, int64_t lddn, int64_t rows, const int32_t *__restrict__ slot_of,
    const float *__restrict__ weights, int64_t tokens, int topk, int64_t hidden,
    float *__restrict__ y, int64_t ldy)
{
    const int64_t quads = hidden / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= tokens * quads)
        return;
    const int64_t t = gid / quads, c = (gid - t * quads) * 4;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int j = 0; j < topk; j++) {
        int64_t s = slot_of[t * topk + j];
        s = s < 0 ? 0 : (s >= rows ? rows - 1 : s);
        const float w = weights[t * topk + j];
        const float4 d = *reinterpret_cast<const float4 *>(dn + s * lddn + c);
        acc.x = __builtin_fmaf(w, d.x, acc.x);
        acc.y = __builtin_fmaf(w, d.y, acc.y);
        acc.z = __builtin_fmaf(w, d.z, acc.z);
        acc.w = __builtin_fmaf(w, d.w, acc.w);
    }
    *reinterpret_cast<float4 *>(y + t * ldy + c) = acc;
}

} // namespace

hipError_t launch_route_sort(const int32_t *expert_of, int64_t tokens, int64_t topk,
                             int64_t experts, int32_t *offsets, int32_t *row_token,
                             int32_t *slot_of, hipStream_t stream)
{
    route_sort_kernel<<<dim3((unsigned)experts), kSortThreads, 0, stream>>>(
        expert_of, (int)(tokens * topk), (int)topk, (int)experts, offsets, row_token, slot_of);
    return hipGetLastError();
}

hipError_t launch_combine(const float *dn, int64_t lddn, int64_t rows, const int32_t *slot_of,
                          const float *weights, int64_t tokens, int64_t topk, int64_t hidden,
                          float *y, int64_t ldy, hipStream_t stream)
{
    const int64_t threads = tokens * (hidden / 4);
    if (threads == 0)
        return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    combine_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(dn, lddn, rows, slot_of, weights,
                                                               tokens, (int)topk, hidden, y, ldy);
    return hipGetLastError();
}

} // namespace bpg
