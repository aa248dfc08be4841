// internal.h -- launchers shared between the C-ABI layer and the kernels.
// Not part of the public interface (see include/bpg.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpg {

// Rotation + quantization of activations; dtype 0 = fp32, 1 = bf16 bits;
// rot = span of the rotation (0: none, 32, 64, 128; k a multiple of it).
hipError_t launch_quantize(const void *x, int dtype, int64_t m, int64_t k, int64_t ldx,
                           int act_bits, int rot, void *codes, float *scales,
                           hipStream_t stream);
// h = silu(gate) * up from gu [rows][ldgu] (gate: columns [0, inter), up:
// [inter, 2 inter)), then rotation + quantization of h.
hipError_t launch_swiglu_quantize(const float *gu, int64_t rows, int64_t inter, int64_t ldgu,
                                  int act_bits, void *codes, float *scales, hipStream_t stream);
// Expert sort of routed rows and the weighted combine (moe.hip).
hipError_t launch_route_sort(const int32_t *expert_of, int64_t tokens, int64_t topk,
                             int64_t experts, int32_t *offsets, int32_t *row_token,
                             int32_t *slot_of, hipStream_t stream);
hipError_t launch_combine(const float *dn, int64_t lddn, int64_t rows, const int32_t *slot_of,
                          const float *weights, int64_t tokens, int64_t topk, int64_t hidden,
                          float *y, int64_t ldy, hipStream_t stream);

// Arguments common to the dense, grouped and block-sum launches.
struct GemmProblem {
    const uint8_t *codes;    // activation codes, [rows][k/2] (4-bit) or [rows][k] (8-bit)
    const float *scales;     // [rows][k/32]
    const uint8_t *wcodes;   // image codes region
    const uint16_t *wscales; // image scales region (fp16 bits)
    int64_t rows;            // activation rows
    int64_t n, k, experts;
    int act_bits;
    // dense / grouped output: fp32 y, or bf16 (round to nearest even) y16
    // when y16 is set; [rows][ldy] elements
    float *y;
    uint16_t *y16;
    int64_t ldy;
    const int32_t *offsets;  // grouped only: [experts+1] on the device
    // grouped only, optional: sorted row r reads activation row row_ids[r]
    // (clamped to [0, src_rows)) instead of row r
    const int32_t *row_ids;
    int64_t src_rows;
    // block sums
    int32_t *sums;
    int64_t m0, m1, n0, n1, expert;
};

// The kernels a product can run.  plan_gemm / plan_grouped_gemm name the one
// launch_gemm / launch_grouped_gemm launch for a problem (host-only, from the
// shape and code width); kernel_name gives its printable name.
enum Kernel {
    kNoKernel = 0,
    kSkinny,       // weight-stream kernel, M <= 32 (skinny.hip)
    kWide,         // 64 x 160 direct-load tiles, 4-bit (wide.hip)
    kStrip,        // 32 x 128 strips (strip.hip)
    kTiled64x160,  // tiled kernel shapes (gemm.hip)
    kTiled64x128,
    kTiled64x64,
    kTiled64x32,
    kTiled16x64,
    kTiled16x32,
    kSlot,         // grouped, 64-row expert slots, 4-bit (grouped.hip)
    kGrouped128,   // grouped tiled kernel, 32-row slots (gemm.hip)
    kGrouped64,
    kGrouped32,
};
int plan_gemm(const GemmProblem &p);
int plan_grouped_gemm(const GemmProblem &p);
const char *kernel_name(int kernel);

hipError_t launch_gemm(const GemmProblem &p, hipStream_t stream);
// The weight-stream kernel for a few rows (dense only): usable when
// skinny_fits(p).
bool skinny_fits(const GemmProblem &p);
hipError_t launch_skinny(const GemmProblem &p, hipStream_t stream);
// The wide-tile kernel (4-bit activations, dense, many rows): 64 x 160
// tiles; usable when wide_fits(p).
bool wide_fits(const GemmProblem &p);
hipError_t launch_wide(const GemmProblem &p, hipStream_t stream);
// The strip kernel (4- or 8-bit activations, dense): 32 x 128 tiles, one
// 32-column tile per wave over all of K; usable when strip_fits(p).
bool strip_fits(const GemmProblem &p);
hipError_t launch_strip(const GemmProblem &p, hipStream_t stream);
// The grouped kernel on 64-row expert slots (4-bit activations, n a multiple
// of 128, at most 1024 experts): usable when grouped_wide_fits(p).
bool grouped_wide_fits(const GemmProblem &p);
hipError_t launch_grouped_wide(const GemmProblem &p, hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmProblem &p, hipStream_t stream);
hipError_t launch_blocksums(const GemmProblem &p, hipStream_t stream);

} // namespace bpg
