// Cache write for new tokens: the indexer key and the latent row.
//
// (GitHub issue "rtx6kpro #90": the "Indexer:" bullet puts the indexer key
// through a LayerNorm with bias whose eps is the model's RMS-norm eps; the
// RoPE bullet makes the rotary embedding interleaved -- entries 2i and 2i+1
// form a pair, not i and i + D/2 as in NeoX style; the first paragraph fixes
// the latent row as 512 latent entries followed by 64 RoPE entries.)
//
// One wave per token, four tokens per workgroup.
//  key    lane l holds the pair (2l, 2l+1) of the D_I entries; mean and
//         variance are wave sums (an xor butterfly, so every lane gets the
//         same bits); the trailing D_rope entries rotate when asked; each value
//         is cast to fp8 e4m3fn (nearest, ties to even, saturating at 448) and
//         the pair's two codes are stored as one 16-bit word.
//  latent the leading D_qk - D_rope entries are copied in 16-byte chunks;
//         lane l < D_rope/2 rotates pair l of the trailing span and rounds to
//         bf16 (nearest even).
// Both parts read the same row of the rotary table.
#include "kernels.h"

namespace ic {
namespace {

constexpr int kWriteThreads = 256;
constexpr int kWriteTokens = kWriteThreads / 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);                 // round to nearest even
    return u >> 16;
}

// fp8 e4m3fn code of an fp32 value: nearest code, ties to even mantissa;
// magnitudes from 448 up take 448 (code 0x7E: the format has no infinity);
// NaN gives 0x7F. The sign bit is kept.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t b = u & 0x7FFFFFFFu;
    const float a = __uint_as_float(b);
    uint32_t m;
    if (!(a < 448.0f))
        m = (a != a) ? 0x7Fu : 0x7Eu;
    else if (a < 0.015625f)                          // below 2^-6: subnormal codes m * 2^-9
        m = (uint32_t)rintf(a * 512.0f);             // 8 lands on 0x08, the smallest normal
    else                                             // keep 3 mantissa bits, rebias exponent 127 -> 7
        m = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    return sign | m;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

__global__ __launch_bounds__(kWriteThreads) void write_cache_kernel(
    const int64_t *__restrict__ row, const int32_t *__restrict__ pos, int32_t T, int64_t rows,
    const float *__restrict__ rope, int64_t n_pos, int32_t D_rope, int32_t key_rope,
    const uint16_t *__restrict__ k_pre, const float *__restrict__ ln_w, const float *__restrict__ ln_b, float eps,
    int32_t D_I, uint8_t *__restrict__ k_idx, const uint16_t *__restrict__ kv_pre, int32_t D_qk,
    uint16_t *__restrict__ kv)
{
    const int t = blockIdx.x * kWriteTokens + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T)
        return;
    const int64_t r = row[t];
    const int32_t p = pos[t];
    // the token's own inputs do not depend on row and pos: load them first so
    // that the wave waits for one round trip before the table read
    const bool kon = k_pre && lane < (D_I >> 1);
    const int half = D_rope >> 1;
    const int lat = D_qk - D_rope;                       // a multiple of 8
    const uint16_t *src = kv_pre + (int64_t)t * D_qk;
    uint32_t kw = 0, rw = 0;
    uint4 c0 = make_uint4(0, 0, 0, 0);
    float2 wv = make_float2(0.f, 0.f), bv = make_float2(0.f, 0.f);
    if (kon) {
        kw = *reinterpret_cast<const uint32_t *>(k_pre + (int64_t)t * D_I + 2 * lane);
        wv = reinterpret_cast<const float2 *>(ln_w)[lane];
        bv = reinterpret_cast<const float2 *>(ln_b)[lane];
    }
    if (kv_pre && lane < (lat >> 3))
        c0 = reinterpret_cast<const uint4 *>(src)[lane];
    if (kv_pre && lane < half)
        rw = *reinterpret_cast<const uint32_t *>(src + lat + 2 * lane);
    // a token whose row or position is out of range writes nothing
    if (r < 0 || r >= rows || (D_rope > 0 && (p < 0 || p >= n_pos)))
        return;
    const float *cs = rope + (int64_t)(D_rope > 0 ? p : 0) * D_rope;

    if (k_pre) {
        const float x0 = bf16_lo(kw), x1 = bf16_hi(kw);  // zero on lanes past D_I / 2
        const float inv_n = 1.0f / (float)D_I;          // D_I is a power of two: exact
        const float mean = wave_sum(x0 + x1) * inv_n;
        const float d0 = kon ? x0 - mean : 0.f, d1 = kon ? x1 - mean : 0.f;
        const float var = wave_sum(d0 * d0 + d1 * d1) * inv_n;
        const float inv = 1.0f / sqrtf(var + eps);
        if (kon) {
            float y0 = d0 * inv * wv.x + bv.x;
            float y1 = d1 * inv * wv.y + bv.y;
            const int i = lane - ((D_I - D_rope) >> 1);  // pair index inside the rotated span
            if (key_rope && i >= 0) {
                const float c = cs[i], s = cs[half + i];
                const float r0 = y0 * c - y1 * s;
                const float r1 = y1 * c + y0 * s;
                y0 = r0;
                y1 = r1;
            }
            *reinterpret_cast<uint16_t *>(k_idx + r * D_I + 2 * lane) =
                (uint16_t)(f32_to_e4m3fn(y0) | (f32_to_e4m3fn(y1) << 8));
        }
    }
    if (kv_pre) {
        uint16_t *dst = kv + r * D_qk;
        if (lane < (lat >> 3))
            reinterpret_cast<uint4 *>(dst)[lane] = c0;
        for (int c = lane + 64; c < (lat >> 3); c += 64)
            reinterpret_cast<uint4 *>(dst)[c] = reinterpret_cast<const uint4 *>(src)[c];
        if (lane < half) {
            const float x0 = bf16_lo(rw), x1 = bf16_hi(rw);
            const float c = cs[lane], s = cs[half + lane];
            const float r0 = x0 * c - x1 * s;
            const float r1 = x1 * c + x0 * s;
            *reinterpret_cast<uint32_t *>(dst + lat + 2 * lane) = f32_to_bf16(r0) | (f32_to_bf16(r1) << 16);
        }
    }
}

}  // namespace

hipError_t launch_write_cache(const int64_t *row, const int32_t *pos, int32_t T, int64_t rows, const float *rope,
                              int64_t n_pos, int32_t D_rope, int32_t key_rope, const uint16_t *k_pre,
                              const float *ln_w, const float *ln_b, float eps, int32_t D_I, uint8_t *k_idx,
                              const uint16_t *kv_pre, int32_t D_qk, uint16_t *kv, hipStream_t stream)
{
    if (T <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((T + kWriteTokens - 1) / kWriteTokens));
    if (!trace_skip("write_cache_kernel"))
        hipLaunchKernelGGL(write_cache_kernel, grid, dim3(kWriteThreads), 0, stream, row, pos, T, rows, rope, n_pos,
                       D_rope, key_rope, k_pre, ln_w, ln_b, eps, D_I, k_idx, kv_pre, D_qk, kv);
    trace_launch(stream, "write_cache_kernel");
    return hipGetLastError();
}

}  // namespace ic
