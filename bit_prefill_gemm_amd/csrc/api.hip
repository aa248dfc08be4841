// api.hip -- the C ABI declared in include/bpg.h.
//
// Every entry point validates its arguments and the weight stamp on the host
// first (so each error except DEVICE / LAUNCH is reported without touching a
// GPU), then checks that the current device is a gfx950, then enqueues its
// kernels on the caller's stream.  rotate_pack_weights runs on the CPU only.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "bpg.h"
#include "internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxGemmK = (int64_t)1 << 22;
std::atomic<int> g_device_ok[kMaxDevices]; // 0 unknown, 1 gfx950, 2 other

bpg_status check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return BPG_ERR_DEVICE;
    if (dev < kMaxDevices) {
        int s = g_device_ok[dev].load(std::memory_order_relaxed);
        if (s == 1)
            return BPG_OK;
        if (s == 2)
            return BPG_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return BPG_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? BPG_OK : BPG_ERR_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// expert sort: one workgroup per expert, each reading every entry (sized for
// prompt batches)
constexpr int64_t kMaxSortExperts = 512;
constexpr int64_t kMaxSortEntries = (int64_t)1 << 20;

bpg_status launch_status(hipError_t e) { return e == hipSuccess ? BPG_OK : BPG_ERR_LAUNCH; }

// groups of four blocks per row
int64_t block_groups(int64_t k) { return (k / 32 + 3) / 4; }

uint64_t image_bytes(int64_t n, int64_t k, int64_t e)
{
    return (uint64_t)e * (uint64_t)(n / 32) * (uint64_t)block_groups(k) * 2304u;
}

// the scales of a group sit after its 2048 code bytes, inside its 2304-byte block
uint64_t scales_offset(int64_t n, int64_t k, int64_t e)
{
    (void)n;
    (void)k;
    (void)e;
    return 2048u;
}

bool shape_ok(int64_t n, int64_t k, int64_t e)
{
    if (n <= 0 || k <= 0 || e <= 0 || n % 32 != 0 || k % 32 != 0)
        return false;
    // keep every byte offset of the image inside int64 and every tile count in int
    if (n > (int64_t)1 << 30 || k > (int64_t)1 << 30 || e > (int64_t)1 << 20)
        return false;
    const long double bytes = (long double)e * (n / 32) * block_groups(k) * 2304;
    return bytes < (long double)((uint64_t)1 << 62);
}

// The stamp check: the analogue of refusing a file that is not a rotated one
// ("509 tokens a second of prompt: the Hadamard route ships", section "Making
// the file is part of the engine").
bpg_status check_stamp(const bpg_weights_desc *w, uint32_t rotation = 32)
{
    if (w->magic != BPG_WEIGHTS_MAGIC || w->version != BPG_WEIGHTS_VERSION ||
        w->rotation != rotation || w->layout != BPG_LAYOUT_GROUP4)
        return BPG_ERR_STAMP;
    if (!shape_ok(w->n, w->k, w->num_experts))
        return BPG_ERR_STAMP;
    if (w->bytes != image_bytes(w->n, w->k, w->num_experts) ||
        w->scales_offset != scales_offset(w->n, w->k, w->num_experts))
        return BPG_ERR_STAMP;
    return BPG_OK;
}

bpg_status check_act(const void *codes, const float *scales, int act_bits, int64_t rows,
                     int64_t k)
{
    if (act_bits != 4 && act_bits != 8)
        return BPG_ERR_DTYPE;
    if (rows < 0 || rows > ((int64_t)1 << 31) - 1)
        return BPG_ERR_SHAPE;
    // with no rows nothing is read, and empty tensors may carry NULL pointers
    if (rows > 0 && (!codes || !scales))
        return BPG_ERR_NULL;
    if (!aligned16(codes) || !aligned16(scales))
        return BPG_ERR_ALIGN;
    // the products address one workgroup's operands with 32-bit offsets
    if (k > kMaxGemmK)
        return BPG_ERR_SHAPE;
    return BPG_OK;
}

// ---------------------------------------------------------------- host packer

// fp64 -> fp16 bits, round to nearest even (the compiler's conversion through
// _Float16 is IEEE round-to-nearest-even on this host).
uint16_t f64_to_f16_bits(double v)
{
    _Float16 h = (_Float16)v;
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

double f16_bits_to_f64(uint16_t b)
{
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (double)h;
}

// In-place fp64 Walsh-Hadamard butterflies over a span of n = 32, 64 or 128
// values, stages h = 1 .. n/2, then times fp64 1/sqrt(n) ("509 tokens a
// second of prompt: the Hadamard route ships", section "The rotation": the
// weights get the same transform, once, offline; spans longer than 32 are the
// "rotations larger than 32" of "Qwen3.8-27B at 45.7 tok/s", "What's next").
void rotate_span_f64(double *v, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int j = 0; j < n; j++)
            if ((j & h) == 0) {
                const double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
    // 1/sqrt(n): sqrt(2)/8, 1/8, sqrt(2)/16 (divisions by powers of two exact)
    const double c = n == 64 ? 0.125 : (n == 128 ? std::sqrt(2.0) / 16.0 : std::sqrt(2.0) / 8.0);
    for (int i = 0; i < n; i++)
        v[i] = v[i] * c;
}

// One Q4_0 block from 32 float weights (already rotated, if at all).
void quantize_weight_block(const double v[32], uint8_t blk[18])
{
    double amax = 0.0;
    for (int i = 0; i < 32; i++)
        amax = std::fabs(v[i]) > amax ? std::fabs(v[i]) : amax;
    const uint16_t hb = f64_to_f16_bits(amax / 7.0);
    const double dw = f16_bits_to_f64(hb);
    blk[0] = (uint8_t)(hb & 0xFF);
    blk[1] = (uint8_t)(hb >> 8);
    int u[32];
    for (int i = 0; i < 32; i++) {
        double q = dw == 0.0 ? 0.0 : std::nearbyint(v[i] / dw);
        q = q < -8.0 ? -8.0 : (q > 7.0 ? 7.0 : q);
        u[i] = (int)q + 8;
    }
    for (int j = 0; j < 16; j++)
        blk[2 + j] = (uint8_t)(u[j] | (u[j + 16] << 4));
}

// Place one canonical 18-byte block of (expert e, row n, block b) in the
// image: its four code dwords go to slots s = 0..3 of its (tile, group)
// block, its scale to the group's scale area (column c = 16h + c16 at
// [c16][h][q]).
inline void place_block(const uint8_t blk[18], int64_t e, int64_t n, int64_t b, int64_t N,
                        int64_t G, uint8_t *img)
{
    uint8_t *grp = img + ((e * (N / 32) + n / 32) * G + b / 4) * 2304;
    const int64_t c = n % 32, q = b % 4;
    for (int s = 0; s < 4; s++)
        std::memcpy(grp + ((s * 32 + c) * 4 + q) * 4, blk + 2 + 4 * s, 4);
    std::memcpy(grp + 2048 + (((c % 16) * 2 + c / 16) * 4 + q) * 2, blk, 2);
}

} // namespace

extern "C" {

const char *bpg_status_str(bpg_status s)
{
    switch (s) {
    case BPG_OK: return "ok";
    case BPG_ERR_NULL: return "null pointer";
    case BPG_ERR_SHAPE: return "invalid shape";
    case BPG_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case BPG_ERR_DTYPE: return "unsupported dtype, source kind or act_bits";
    case BPG_ERR_STAMP: return "weight image stamp missing, foreign, of the other route or inconsistent";
    case BPG_ERR_BUFFER: return "destination buffer too small";
    case BPG_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case BPG_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

size_t rotate_pack_weights_bytes(int64_t n, int64_t k, int64_t num_experts)
{
    if (!shape_ok(n, k, num_experts))
        return 0;
    return (size_t)image_bytes(n, k, num_experts);
}

} // extern "C"

namespace {

// The packer of every route: rot = 32 (or 64, 128) makes a rotated image
// (stamp rotation rot; sources: float weights, rotated on the way, or the
// Q4_0 tensors of a file rotated that way), rot = 0 the unrotated one (stamp
// rotation 0; sources: float weights or plain Q4_0 tensors).
bpg_status pack_image(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                      int64_t num_experts, void *dst_host, size_t dst_bytes,
                      bpg_weights_desc *desc_out, int rot)
{
    const bpg_src_kind q4_kind = rot ? BPG_SRC_Q4_0_ROTATED : BPG_SRC_Q4_0;
    if (kind != BPG_SRC_F32 && kind != BPG_SRC_BF16 && kind != q4_kind)
        return BPG_ERR_DTYPE;
    if (!shape_ok(n, k, num_experts) || k % (rot > 32 ? rot : 32) != 0)
        return BPG_ERR_SHAPE;
    if (!src || !dst_host || !desc_out)
        return BPG_ERR_NULL;
    const uint64_t total = image_bytes(n, k, num_experts);
    if (dst_bytes < total)
        return BPG_ERR_BUFFER;

    const int64_t B = k / 32, G = block_groups(k);
    uint8_t *img = static_cast<uint8_t *>(dst_host);
    // blocks past B: codes 0x88 (value 0), scale 0
    for (uint64_t off = 0; off < total; off += 2304) {
        std::memset(img + off, 0x88, 2048);
        std::memset(img + off + 2048, 0, 256);
    }
    const int span = rot > 32 ? rot : 32; // values rotated together
    for (int64_t e = 0; e < num_experts; e++)
        for (int64_t r = 0; r < n; r++) {
            const int64_t row = e * n + r;
            for (int64_t s0 = 0; s0 < B; s0 += span / 32) {
                double v[128];
                if (kind != q4_kind) {
                    for (int i = 0; i < span; i++) {
                        const int64_t idx = row * k + s0 * 32 + i;
                        if (kind == BPG_SRC_F32) {
                            v[i] = (double)static_cast<const float *>(src)[idx];
                        } else {
                            const uint32_t bits = (uint32_t)static_cast<const uint16_t *>(src)[idx] << 16;
                            float f;
                            std::memcpy(&f, &bits, 4);
                            v[i] = (double)f;
                        }
                    }
                    if (rot)
                        rotate_span_f64(v, span);
                }
                for (int64_t b = s0; b < s0 + span / 32; b++) {
                    uint8_t blk[18];
                    if (kind == q4_kind)
                        std::memcpy(blk, static_cast<const uint8_t *>(src) + (row * B + b) * 18, 18);
                    else
                        quantize_weight_block(v + (b - s0) * 32, blk);
                    place_block(blk, e, r, b, n, G, img);
                }
            }
        }

    bpg_weights_desc d;
    std::memset(&d, 0, sizeof d);
    d.magic = BPG_WEIGHTS_MAGIC;
    d.version = BPG_WEIGHTS_VERSION;
    d.rotation = (uint32_t)rot;
    d.layout = BPG_LAYOUT_GROUP4;
    d.n = n;
    d.k = k;
    d.num_experts = num_experts;
    d.bytes = total;
    d.scales_offset = scales_offset(n, k, num_experts);
    *desc_out = d;
    return BPG_OK;
}

// rot: span of the rotation (0 = none, 32, 64, 128)
bpg_status quantize_checked(const void *x, bpg_x_dtype dt, int64_t m, int64_t k, int64_t ldx,
                            int act_bits, void *codes, float *scales, void *stream, int rot)
{
    if (dt != BPG_X_F32 && dt != BPG_X_BF16)
        return BPG_ERR_DTYPE;
    if (act_bits != 4 && act_bits != 8)
        return BPG_ERR_DTYPE;
    if (m < 0 || k <= 0 || k % (rot > 32 ? rot : 32) != 0 || ldx < k || m > ((int64_t)1 << 31) - 1 ||
        k > ((int64_t)1 << 30) || ldx > ((int64_t)1 << 40))
        return BPG_ERR_SHAPE;
    if (m > 0 && (!x || !codes || !scales))
        return BPG_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || ldx % 4 != 0)
        return BPG_ERR_ALIGN;
    bpg_status s = check_device();
    if (s != BPG_OK)
        return s;
    return launch_status(bpg::launch_quantize(x, (int)dt, m, k, ldx, act_bits, rot, codes,
                                              scales, static_cast<hipStream_t>(stream)));
}

// y: fp32 [m][ldy], or bf16 bits when y_bf16 (rows 16-byte aligned either way)
bpg_status gemm_checked(const void *codes, const float *scales, int act_bits, int64_t m,
                        const bpg_weights_desc *w, const void *w_dev, void *y, bool y_bf16,
                        int64_t ldy, void *stream, uint32_t rotation)
{
    if (!w)
        return BPG_ERR_NULL;
    bpg_status s = check_stamp(w, rotation);
    if (s != BPG_OK)
        return s;
    if (w->num_experts != 1)
        return BPG_ERR_STAMP;
    s = check_act(codes, scales, act_bits, m, w->k);
    if (s != BPG_OK)
        return s;
    if (ldy < w->n)
        return BPG_ERR_SHAPE;
    if (!w_dev || (m > 0 && !y))
        return BPG_ERR_NULL;
    if (!aligned16(w_dev) || !aligned16(y) || ldy % (y_bf16 ? 8 : 4) != 0)
        return BPG_ERR_ALIGN;
    s = check_device();
    if (s != BPG_OK)
        return s;
    bpg::GemmProblem p{};
    p.codes = static_cast<const uint8_t *>(codes);
    p.scales = scales;
    p.wcodes = static_cast<const uint8_t *>(w_dev);
    p.wscales = reinterpret_cast<const uint16_t *>(p.wcodes + w->scales_offset);
    p.rows = m;
    p.n = w->n;
    p.k = w->k;
    p.experts = 1;
    p.act_bits = act_bits;
    if (y_bf16)
        p.y16 = static_cast<uint16_t *>(y);
    else
        p.y = static_cast<float *>(y);
    p.ldy = ldy;
    return launch_status(bpg::launch_gemm(p, static_cast<hipStream_t>(stream)));
}

} // namespace

extern "C" {

bpg_status rotate_pack_weights(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                               int64_t num_experts, void *dst_host, size_t dst_bytes,
                               bpg_weights_desc *desc_out)
{
    return pack_image(src, kind, n, k, num_experts, dst_host, dst_bytes, desc_out, 32);
}

bpg_status pack_weights_unrotated(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                                  int64_t num_experts, void *dst_host, size_t dst_bytes,
                                  bpg_weights_desc *desc_out)
{
    return pack_image(src, kind, n, k, num_experts, dst_host, dst_bytes, desc_out, 0);
}

bpg_status quantize_act_h32(const void *x, bpg_x_dtype dt, int64_t m, int64_t k, int64_t ldx,
                            int act_bits, void *codes, float *scales, void *stream)
{
    return quantize_checked(x, dt, m, k, ldx, act_bits, codes, scales, stream, 32);
}

bpg_status quantize_act_unrotated(const void *x, bpg_x_dtype dt, int64_t m, int64_t k,
                                  int64_t ldx, int act_bits, void *codes, float *scales,
                                  void *stream)
{
    return quantize_checked(x, dt, m, k, ldx, act_bits, codes, scales, stream, 0);
}

bpg_status w4a4_gemm(const void *codes, const float *scales, int act_bits, int64_t m,
                     const bpg_weights_desc *w, const void *w_dev, float *y, int64_t ldy,
                     void *stream)
{
    return gemm_checked(codes, scales, act_bits, m, w, w_dev, y, false, ldy, stream, 32);
}

bpg_status w4a4_gemm_bf16(const void *codes, const float *scales, int act_bits, int64_t m,
                          const bpg_weights_desc *w, const void *w_dev, uint16_t *y, int64_t ldy,
                          void *stream)
{
    return gemm_checked(codes, scales, act_bits, m, w, w_dev, y, true, ldy, stream, 32);
}

bpg_status w4a4_gemm_unrotated(const void *codes, const float *scales, int act_bits, int64_t m,
                               const bpg_weights_desc *w, const void *w_dev, float *y,
                               int64_t ldy, void *stream)
{
    return gemm_checked(codes, scales, act_bits, m, w, w_dev, y, false, ldy, stream, 0);
}

bpg_status rotate_pack_weights_rot(const void *src, bpg_src_kind kind, int64_t n, int64_t k,
                                   int64_t num_experts, int rotation, void *dst_host,
                                   size_t dst_bytes, bpg_weights_desc *desc_out)
{
    if (rotation != 32 && rotation != 64 && rotation != 128)
        return BPG_ERR_SHAPE;
    return pack_image(src, kind, n, k, num_experts, dst_host, dst_bytes, desc_out, rotation);
}

bpg_status quantize_act_rot(const void *x, bpg_x_dtype dt, int64_t m, int64_t k, int64_t ldx,
                            int act_bits, int rotation, void *codes, float *scales, void *stream)
{
    if (rotation != 32 && rotation != 64 && rotation != 128)
        return BPG_ERR_SHAPE;
    return quantize_checked(x, dt, m, k, ldx, act_bits, codes, scales, stream, rotation);
}

const char *w4a4_gemm_kernel_name(int act_bits, int64_t m, const bpg_weights_desc *w)
{
    if (!w || (act_bits != 4 && act_bits != 8) || m < 0 || m > ((int64_t)1 << 31) - 1)
        return nullptr;
    if (check_stamp(w, w->rotation) != BPG_OK || w->num_experts != 1)
        return nullptr;
    bpg::GemmProblem p{};
    p.rows = m;
    p.n = w->n;
    p.k = w->k;
    p.experts = 1;
    p.act_bits = act_bits;
    return bpg::kernel_name(bpg::plan_gemm(p));
}

const char *w4a4_grouped_gemm_kernel_name(int act_bits, int64_t total_rows, int64_t src_rows,
                                          const bpg_weights_desc *w)
{
    if (!w || (act_bits != 4 && act_bits != 8) || total_rows < 0 ||
        total_rows > ((int64_t)1 << 31) - 1 || src_rows < 0)
        return nullptr;
    if (check_stamp(w) != BPG_OK)
        return nullptr;
    static const int32_t kNotRead = 0; // stands for a row index: only tested for presence
    bpg::GemmProblem p{};
    p.rows = total_rows;
    p.n = w->n;
    p.k = w->k;
    p.experts = w->num_experts;
    p.act_bits = act_bits;
    p.row_ids = src_rows > 0 ? &kNotRead : nullptr;
    p.src_rows = src_rows;
    return bpg::kernel_name(bpg::plan_grouped_gemm(p));
}

bpg_status w4a4_gemm_rot(const void *codes, const float *scales, int act_bits, int rotation,
                         int64_t m, const bpg_weights_desc *w, const void *w_dev, float *y,
                         int64_t ldy, void *stream)
{
    if (rotation != 32 && rotation != 64 && rotation != 128)
        return BPG_ERR_SHAPE;
    return gemm_checked(codes, scales, act_bits, m, w, w_dev, y, false, ldy, stream, (uint32_t)rotation);
}

} // extern "C"

namespace {

// gather: rows are read through row_ids (src_rows activation rows)
bpg_status grouped_checked(const void *codes, const float *scales, int act_bits, bool gather,
                           int64_t src_rows, const int32_t *row_ids, int64_t total_rows,
                           const int32_t *expert_offsets_dev, const bpg_weights_desc *w,
                           const void *w_dev, void *y, bool y_bf16, int64_t ldy, void *stream)
{
    if (!w)
        return BPG_ERR_NULL;
    bpg_status s = check_stamp(w);
    if (s != BPG_OK)
        return s;
    if (total_rows < 0 || total_rows > ((int64_t)1 << 31) - 1)
        return BPG_ERR_SHAPE;
    s = check_act(codes, scales, act_bits, gather ? src_rows : total_rows, w->k);
    if (s != BPG_OK)
        return s;
    if (gather) {
        if (src_rows < 0)
            return BPG_ERR_SHAPE;
        if (total_rows > 0 && !row_ids)
            return BPG_ERR_NULL;
        // gathered rows are addressed from row 0 with 32-bit offsets
        const int64_t row_bytes = w->k * (act_bits == 4 ? 16 : 32) / 32;
        if (total_rows > 0 && src_rows == 0)
            return BPG_ERR_SHAPE;
        if (src_rows * row_bytes >= ((int64_t)1 << 31) || src_rows * (w->k / 32) >= ((int64_t)1 << 31))
            return BPG_ERR_SHAPE;
    }
    if (ldy < w->n)
        return BPG_ERR_SHAPE;
    if (!w_dev || !expert_offsets_dev || (total_rows > 0 && !y))
        return BPG_ERR_NULL;
    if (!aligned16(w_dev) || !aligned16(y) || ldy % (y_bf16 ? 8 : 4) != 0 ||
        (reinterpret_cast<uintptr_t>(expert_offsets_dev) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(row_ids) & 3u) != 0)
        return BPG_ERR_ALIGN;
    s = check_device();
    if (s != BPG_OK)
        return s;
    bpg::GemmProblem p{};
    p.codes = static_cast<const uint8_t *>(codes);
    p.scales = scales;
    p.wcodes = static_cast<const uint8_t *>(w_dev);
    p.wscales = reinterpret_cast<const uint16_t *>(p.wcodes + w->scales_offset);
    p.rows = total_rows;
    p.n = w->n;
    p.k = w->k;
    p.experts = w->num_experts;
    p.act_bits = act_bits;
    if (y_bf16)
        p.y16 = static_cast<uint16_t *>(y);
    else
        p.y = static_cast<float *>(y);
    p.ldy = ldy;
    p.offsets = expert_offsets_dev;
    p.row_ids = gather ? row_ids : nullptr;
    p.src_rows = src_rows;
    return launch_status(bpg::launch_grouped_gemm(p, static_cast<hipStream_t>(stream)));
}

} // namespace

extern "C" {

bpg_status w4a4_grouped_gemm(const void *codes, const float *scales, int act_bits,
                             int64_t total_rows, const int32_t *expert_offsets_dev,
                             const bpg_weights_desc *w, const void *w_dev, float *y,
                             int64_t ldy, void *stream)
{
    return grouped_checked(codes, scales, act_bits, false, total_rows, nullptr, total_rows,
                           expert_offsets_dev, w, w_dev, y, false, ldy, stream);
}

bpg_status w4a4_grouped_gemm_bf16(const void *codes, const float *scales, int act_bits,
                                  int64_t total_rows, const int32_t *expert_offsets_dev,
                                  const bpg_weights_desc *w, const void *w_dev, uint16_t *y,
                                  int64_t ldy, void *stream)
{
    return grouped_checked(codes, scales, act_bits, false, total_rows, nullptr, total_rows,
                           expert_offsets_dev, w, w_dev, y, true, ldy, stream);
}

bpg_status w4a4_grouped_gemm_gather(const void *codes, const float *scales, int act_bits,
                                    int64_t src_rows, const int32_t *row_ids_dev,
                                    int64_t total_rows, const int32_t *expert_offsets_dev,
                                    const bpg_weights_desc *w, const void *w_dev, float *y,
                                    int64_t ldy, void *stream)
{
    return grouped_checked(codes, scales, act_bits, true, src_rows, row_ids_dev, total_rows,
                           expert_offsets_dev, w, w_dev, y, false, ldy, stream);
}

bpg_status moe_route_sort(const int32_t *expert_of_dev, int64_t tokens, int64_t topk,
                          int64_t experts, int32_t *offsets_dev, int32_t *row_token_dev,
                          int32_t *slot_of_dev, void *stream)
{
    if (tokens < 0 || topk < 1 || experts < 1 || experts > kMaxSortExperts ||
        tokens * topk > kMaxSortEntries)
        return BPG_ERR_SHAPE;
    if (!offsets_dev || (tokens > 0 && (!expert_of_dev || !row_token_dev || !slot_of_dev)))
        return BPG_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(expert_of_dev) | reinterpret_cast<uintptr_t>(offsets_dev) |
          reinterpret_cast<uintptr_t>(row_token_dev) | reinterpret_cast<uintptr_t>(slot_of_dev)) &
         3u) != 0)
        return BPG_ERR_ALIGN;
    bpg_status s = check_device();
    if (s != BPG_OK)
        return s;
    return launch_status(bpg::launch_route_sort(expert_of_dev, tokens, topk, experts, offsets_dev,
                                                row_token_dev, slot_of_dev,
                                                static_cast<hipStream_t>(stream)));
}

bpg_status swiglu_quantize_h32(const float *gu, int64_t rows, int64_t inter, int64_t ldgu,
                               int act_bits, void *codes, float *scales, void *stream)
{
    if (act_bits != 4 && act_bits != 8)
        return BPG_ERR_DTYPE;
    if (rows < 0 || inter <= 0 || inter % 32 != 0 || ldgu < 2 * inter ||
        rows > ((int64_t)1 << 31) - 1 || inter > ((int64_t)1 << 30) || ldgu > ((int64_t)1 << 40))
        return BPG_ERR_SHAPE;
    if (rows > 0 && (!gu || !codes || !scales))
        return BPG_ERR_NULL;
    if (!aligned16(gu) || !aligned16(codes) || !aligned16(scales) || ldgu % 4 != 0)
        return BPG_ERR_ALIGN;
    bpg_status s = check_device();
    if (s != BPG_OK)
        return s;
    return launch_status(bpg::launch_swiglu_quantize(gu, rows, inter, ldgu, act_bits, codes, scales,
                                                     static_cast<hipStream_t>(stream)));
}

bpg_status moe_combine(const float *dn, int64_t lddn, int64_t rows, const int32_t *slot_of_dev,
                       const float *weights_dev, int64_t tokens, int64_t topk, int64_t hidden,
                       float *y, int64_t ldy, void *stream)
{
    if (tokens < 0 || topk < 1 || hidden <= 0 || hidden % 4 != 0 || lddn < hidden ||
        ldy < hidden || rows < 0 || (tokens > 0 && rows == 0) || tokens * topk > kMaxSortEntries)
        return BPG_ERR_SHAPE;
    if (tokens > 0 && (!dn || !slot_of_dev || !weights_dev || !y))
        return BPG_ERR_NULL;
    if (!aligned16(dn) || !aligned16(y) || lddn % 4 != 0 || ldy % 4 != 0 ||
        ((reinterpret_cast<uintptr_t>(slot_of_dev) | reinterpret_cast<uintptr_t>(weights_dev)) &
         3u) != 0)
        return BPG_ERR_ALIGN;
    bpg_status s = check_device();
    if (s != BPG_OK)
        return s;
    return launch_status(bpg::launch_combine(dn, lddn, rows, slot_of_dev, weights_dev, tokens, topk,
                                             hidden, y, ldy, static_cast<hipStream_t>(stream)));
}

bpg_status w4a4_gemm_blocksums(const void *codes, const float *scales, int act_bits, int64_t m,
                               const bpg_weights_desc *w, const void *w_dev, int64_t expert,
                               int64_t m0, int64_t m1, int64_t n0, int64_t n1, int32_t *sums,
                               void *stream)
{
    if (!w)
        return BPG_ERR_NULL;
    bpg_status s = check_stamp(w);
    if (s != BPG_OK)
        return s;
    if (act_bits != 4 && act_bits != 8)
        return BPG_ERR_DTYPE;
    if (m < 0 || expert < 0 || expert >= w->num_experts || m0 < 0 || m0 > m1 || m1 > m ||
        n0 < 0 || n0 > n1 || n1 > w->n || m > ((int64_t)1 << 31) - 1 || w->k > kMaxGemmK)
        return BPG_ERR_SHAPE;
    if (!codes || !w_dev || !sums)
        return BPG_ERR_NULL;
    if (!aligned16(codes) || !aligned16(w_dev) || !aligned16(sums) ||
        (scales && !aligned16(scales)))
        return BPG_ERR_ALIGN;
    s = check_device();
    if (s != BPG_OK)
        return s;
    bpg::GemmProblem p{};
    p.codes = static_cast<const uint8_t *>(codes);
    p.scales = scales;
    p.wcodes = static_cast<const uint8_t *>(w_dev);
    p.wscales = reinterpret_cast<const uint16_t *>(p.wcodes + w->scales_offset);
    p.rows = m;
    p.n = w->n;
    p.k = w->k;
    p.experts = w->num_experts;
    p.act_bits = act_bits;
    p.sums = sums;
    p.m0 = m0;
    p.m1 = m1;
    p.n0 = n0;
    p.n1 = n1;
    p.expert = expert;
    return launch_status(bpg::launch_blocksums(p, static_cast<hipStream_t>(stream)));
}

} // extern "C"
