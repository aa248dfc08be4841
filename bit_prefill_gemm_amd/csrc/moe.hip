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

constexpr int kSortThreads = 1024;  // one workgroup: 16 waves
constexpr int kSortWaves = kSortThreads / 64;

// Counting sort in one workgroup.  Pass 1 counts the entries per expert (LDS
// atomics: the totals do not depend on their order) and scans the counts into
// offsets.  Pass 2 walks the entries in chunks of 1024, one per thread; inside
// a wave every lane finds how many lower lanes hold its expert with ballots
// (one round per distinct expert in the wave, at most 64), the per-wave
// counts are scanned across the 16 waves per expert, and each entry lands at
// offset + earlier chunks + earlier waves + earlier lanes: the stable order.
// Expert ids outside [0, experts) are clamped (the rows stay in bounds).
__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const int32_t *__restrict__ expert_of, int n, int topk, int experts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ row_token, int32_t *__restrict__ slot_of)
{
    extern __shared__ int32_t sh[];
    int32_t *base = sh;                   // [experts]: next free position
    int32_t *wcnt = sh + experts;         // [kSortWaves][experts]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < experts; e += kSortThreads)
        base[e] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSortThreads) {
        int e = expert_of[i];
        e = e < 0 ? 0 : (e >= experts ? experts - 1 : e);
        atomicAdd(&base[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < experts; e++) {
            const int c = base[e];
            offsets[e] = run;
            base[e] = run;
            run += c;
        }
        offsets[experts] = run;
    }
    __syncthreads();

    for (int c0 = 0; c0 < n; c0 += kSortThreads) {
        for (int i = tid; i < kSortWaves * experts; i += kSortThreads)
            wcnt[i] = 0;
        __syncthreads();
        const int idx = c0 + tid;
        const bool valid = idx < n;
        int e = 0;
        if (valid) {
            e = expert_of[idx];
            e = e < 0 ? 0 : (e >= experts ? experts - 1 : e);
        }
        // rank among the lower lanes of this wave with the same expert
        uint64_t left = __ballot(valid);
        int rank = 0;
        while (left != 0) { // uniform: every lane sees the same mask
            const int leader = __builtin_ctzll(left);
            const int x = __builtin_amdgcn_readlane(e, leader);
            const uint64_t same = __ballot(valid && e == x) & left;
            if (valid && e == x) {
                rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
                if (lane == leader)
                    wcnt[wave * experts + x] = __builtin_popcountll(same);
            }
            left &= ~same;
        }
        __syncthreads();
        // per expert: exclusive scan over the waves, then advance the base
        for (int x = tid; x < experts; x += kSortThreads) {
            int run = base[x];
            for (int w = 0; w < kSortWaves; w++) {
                const int cnt = wcnt[w * experts + x];
                wcnt[w * experts + x] = run;
                run += cnt;
            }
            base[x] = run;
        }
        __syncthreads();
        if (valid) {
            const int pos = wcnt[wave * experts + e] + rank;
            slot_of[idx] = pos;
            row_token[pos] = idx / topk;
        }
        __syncthreads();
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
    const size_t lds = (size_t)(1 + kSortWaves) * experts * sizeof(int32_t);
    route_sort_kernel<<<1, kSortThreads, lds, stream>>>(expert_of, (int)(tokens * topk), (int)topk,
                                                        (int)experts, offsets, row_token, slot_of);
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
