"""MI355X-native (gfx950) Hadamard-rotated W4A4 prompt GEMM.

The route ("509 tokens a second of prompt: the Hadamard route ships"):
rotate each 32-value activation block by a 32-point Walsh-Hadamard transform,
quantize it to 4-bit codes with one scale per block, and multiply the codes
against Q4_0 weights that were rotated the same way offline.

Public names mirror the C ABI in include/bpg.h:

    rotate_pack_weights, quantize_act_h32, w4a4_gemm, w4a4_grouped_gemm,
    w4a4_gemm_blocksums, and the unrotated route's pack_weights_unrotated,
    quantize_act_unrotated, w4a4_gemm_unrotated; and the expert layer's glue:
    moe_route_sort, w4a4_grouped_gemm_gather, swiglu_quantize_h32, moe_combine;
    and rotations over 64 or 128 values: rotate_pack_weights_rot,
    quantize_act_rot, w4a4_gemm_rot; and bf16 output: w4a4_gemm_bf16,
    w4a4_grouped_gemm_bf16

The binding is loaded lazily so that ``bit_prefill_gemm_amd.synth`` (input
generators) imports without the HIP library.
"""
_BINDING_NAMES = {
    "rotate_pack_weights", "rotate_pack_weights_bytes", "quantize_act_h32", "w4a4_gemm",
    "w4a4_grouped_gemm", "w4a4_gemm_blocksums", "Weights", "WeightsDesc", "BpgError",
    "SRC_F32", "SRC_BF16", "SRC_Q4_0_ROTATED", "SRC_Q4_0", "X_F32", "X_BF16",
    "pack_weights_unrotated", "quantize_act_unrotated", "w4a4_gemm_unrotated",
    "moe_route_sort", "w4a4_grouped_gemm_gather", "swiglu_quantize_h32", "moe_combine",
    "rotate_pack_weights_rot", "quantize_act_rot", "w4a4_gemm_rot",
    "w4a4_gemm_bf16", "w4a4_grouped_gemm_bf16",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
