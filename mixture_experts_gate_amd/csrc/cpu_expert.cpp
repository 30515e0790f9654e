// Host side of the bandwidth-adaptive placement: the SwiGLU expert FFN computed
// on the host CPU from an expert blob in pinned host memory, for experts whose
// copy over the host link would take longer than computing them where they
// already are (winzheng.com page, "FreeToken's Three-Layer Mechanism": the
// system measures the bandwidth it actually gets and decides per expert
// whether the GPU or the CPU computes it; aimodeling.com/en page, "Three
// Engineering Cores").
//
// The blob is in the kernel MXFP4 layout (the layout the cache's host store
// holds): each matrix in 16-row x 128-column blocks; in block (rb, s) the 16
// code bytes of "lane" l are row 16rb + l%16, columns 128s + 32(l/16) + 0..31
// (even element in the low nibble), and scale byte l is that run's E8M0 scale.
// Work is split over row blocks; each thread decodes a 16 x 128 block into
// fp32 once and applies it to every token row. Accumulation is fp32; the
// activation is rounded to bf16 between the two contractions and y to bf16,
// as on the GPU's weight-streaming path.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include <immintrin.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#include "moe.h"

namespace {

// E2M1 code -> value (OCP microscaling element grid, sign in bit 3)
const float kE2M1[16] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
                         -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

inline uint16_t f32_to_bf16(float f) {     // round to nearest even (finite inputs)
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

inline float e8m0(uint8_t s) {
    return s ? ldexpf(1.0f, (int)s - 127) : ldexpf(1.0f, -127);
}

// Decode block (rb, s) of a matrix with K columns into w[16][128] (row-major).
inline void decode_block(const uint8_t *codes, const uint8_t *scales, long rb, int s, int nslab,
                         float (*w)[128]) {
    const size_t blk = (size_t)rb * nslab + s;
    const uint8_t *c = codes + blk * 1024;
    const uint8_t *sc = scales + blk * 64;
    for (int l = 0; l < 64; ++l) {
        const int row = l & 15, col = 32 * (l >> 4);
        const float f = e8m0(sc[l]);
        const uint8_t *q = c + 16 * l;
        float *dst = &w[row][col];
        for (int j = 0; j < 16; ++j) {
            dst[2 * j] = kE2M1[q[j] & 15] * f;
            dst[2 * j + 1] = kE2M1[q[j] >> 4] * f;
        }
    }
}

// The same with AVX2: each code becomes twice its E2M1 value as an int8
// through a 16-entry byte table (exact integers -12..12), widened to fp32 and
// multiplied by half the block scale (exact, so the values equal the table
// decode's bit for bit).
__attribute__((target("avx2"))) void decode_block_avx2(const uint8_t *codes,
                                                       const uint8_t *scales, long rb, int s,
                                                       int nslab, float (*w)[128]) {
    const size_t blk = (size_t)rb * nslab + s;
    const uint8_t *c = codes + blk * 1024;
    const uint8_t *sc = scales + blk * 64;
    const __m128i lut = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
    const __m128i m4 = _mm_set1_epi8(0x0F);
    for (int l = 0; l < 64; ++l) {
        const __m256 f = _mm256_set1_ps(0.5f * e8m0(sc[l]));
        const __m128i q = _mm_loadu_si128(reinterpret_cast<const __m128i *>(c + 16 * l));
        const __m128i lo = _mm_shuffle_epi8(lut, _mm_and_si128(q, m4));
        const __m128i hi = _mm_shuffle_epi8(lut, _mm_and_si128(_mm_srli_epi16(q, 4), m4));
        const __m128i v0 = _mm_unpacklo_epi8(lo, hi);   // elements 0..15 (even = low nibble)
        const __m128i v1 = _mm_unpackhi_epi8(lo, hi);   // elements 16..31
        float *dst = &w[l & 15][32 * (l >> 4)];
        _mm256_storeu_ps(dst, _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v0)), f));
        _mm256_storeu_ps(dst + 8, _mm256_mul_ps(
            _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v0, 8))), f));
        _mm256_storeu_ps(dst + 16,
                         _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v1)), f));
        _mm256_storeu_ps(dst + 24, _mm256_mul_ps(
            _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v1, 8))), f));
    }
}

const bool kHostAvx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");

// moe_cpu_block_rows with AVX2 + FMA: per token row, the 16 output rows'
// sums are kept as 8-lane partial vectors across all slabs (one horizontal
// sum per output at the end), each slab's block decoded once for all rows.
__attribute__((target("avx2,fma"))) void block_rows_avx2(const uint8_t *codes,
                                                         const uint8_t *scales, long rb, int K,
                                                         const float *in, int n, float *out,
                                                         int out_stride) {
    const int nslab = K / 128;
    alignas(32) float w[16][128];
    // 8-lane partial sums [n][16][8] (unaligned loads and stores: a vector of
    // __m256 would not keep the type's 32-byte alignment)
    std::vector<float> acc((size_t)n * 16 * 8, 0.0f);
    for (int s = 0; s < nslab; ++s) {
        decode_block_avx2(codes, scales, rb, s, nslab, w);
        for (int r = 0; r < n; ++r) {
            const float *x = in + (size_t)r * K + 128 * s;
            float *a = acc.data() + (size_t)r * 128;
            for (int h = 0; h < 2; ++h) {
                __m256 t[8];
                for (int i = 0; i < 8; ++i) t[i] = _mm256_loadu_ps(a + 8 * (8 * h + i));
                for (int k = 0; k < 128; k += 8) {
                    const __m256 xv = _mm256_loadu_ps(x + k);
                    for (int i = 0; i < 8; ++i)
                        t[i] = _mm256_fmadd_ps(_mm256_load_ps(&w[8 * h + i][k]), xv, t[i]);
                }
                for (int i = 0; i < 8; ++i) _mm256_storeu_ps(a + 8 * (8 * h + i), t[i]);
            }
        }
    }
    for (int r = 0; r < n; ++r)
        for (int i = 0; i < 16; ++i) {
            const __m256 v = _mm256_loadu_ps(acc.data() + ((size_t)r * 16 + i) * 8);
            const __m128 q = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
            const __m128 d = _mm_add_ps(q, _mm_movehl_ps(q, q));
            const __m128 e = _mm_add_ss(d, _mm_shuffle_ps(d, d, 1));
            out[(size_t)r * out_stride + 16 * rb + i] = _mm_cvtss_f32(e);
        }
}

}  // namespace

// out[r][16 rb + i] = sum_k in[r][k] * W[16 rb + i][k] for the 16 rows of row
// block rb, every row r < n (in: fp32 rows of length K). On hosts with AVX2
// and FMA (checked once at load) the vector kernel above runs; elsewhere this
// portable loop (the fp32 sums then add in another order).
void moe_cpu_block_rows(const uint8_t *codes, const uint8_t *scales, long rb, int K,
                       const float *in, int n, float *out, int out_stride) {
    if (kHostAvx2) {
        block_rows_avx2(codes, scales, rb, K, in, n, out, out_stride);
        return;
    }
    const int nslab = K / 128;
    float w[16][128];
    float acc_small[16 * 16];
    std::vector<float> acc_big(n > 16 ? (size_t)n * 16 : 0);
    float *acc = n > 16 ? acc_big.data() : acc_small;
    for (int i = 0; i < n * 16; ++i) acc[i] = 0.0f;
    for (int s = 0; s < nslab; ++s) {
        decode_block(codes, scales, rb, s, nslab, w);
        for (int r = 0; r < n; ++r) {
            const float *x = in + (size_t)r * K + 128 * s;
            float *a = acc + (size_t)r * 16;
            for (int i = 0; i < 16; ++i) {
                float sum = 0.0f;
#pragma omp simd reduction(+ : sum)
                for (int k = 0; k < 128; ++k) sum += w[i][k] * x[k];
                a[i] += sum;
            }
        }
    }
    for (int r = 0; r < n; ++r)
        for (int i = 0; i < 16; ++i) out[(size_t)r * out_stride + 16 * rb + i] = acc[(size_t)r * 16 + i];
}

extern "C" int moe_cpu_expert_ffn(int fmt, const void *w13, const uint8_t *s13, const void *w2,
                                  const uint8_t *s2, int H, int I, const uint16_t *x_rows, int n,
                                  uint16_t *y_rows, int threads) {
    if (fmt != MOE_W_MXFP4) return MOE_EUNSUPPORTED;
    if (H < 128 || I < 128 || H % 128 || I % 128 || n < 0) return MOE_EINVAL;
    if (n == 0) return MOE_OK;
    if (!w13 || !s13 || !w2 || !s2 || !x_rows || !y_rows) return MOE_EINVAL;
    const uint8_t *c13 = static_cast<const uint8_t *>(w13);
    const uint8_t *c2 = static_cast<const uint8_t *>(w2);
    std::vector<float> x((size_t)n * H), gu((size_t)n * 2 * I), a((size_t)n * I),
        y((size_t)n * H);
    for (size_t i = 0; i < x.size(); ++i) x[i] = bf16_to_f32(x_rows[i]);
#ifdef _OPENMP
    const int nt = threads > 0 ? threads : omp_get_max_threads();
#else
    const int nt = 1;
    (void)threads;
#endif
    // gate and up rows: 2I / 16 row blocks over K = H
    const long nb13 = 2L * I / 16;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (long rb = 0; rb < nb13; ++rb) moe_cpu_block_rows(c13, s13, rb, H, x.data(), n, gu.data(), 2 * I);
    for (int r = 0; r < n; ++r)
        for (int i = 0; i < I; ++i) {
            const float g = gu[(size_t)r * 2 * I + i], u = gu[(size_t)r * 2 * I + I + i];
            a[(size_t)r * I + i] = bf16_to_f32(f32_to_bf16(g / (1.0f + expf(-g)) * u));
        }
    // down rows: H / 16 row blocks over K = I
    const long nb2 = (long)H / 16;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (long rb = 0; rb < nb2; ++rb) moe_cpu_block_rows(c2, s2, rb, I, a.data(), n, y.data(), H);
    for (size_t i = 0; i < y.size(); ++i) y_rows[i] = f32_to_bf16(y[i]);
    return MOE_OK;
}

// The permutation restricted to the experts the device computes (the host
// experts' rows removed, their counts zero), and the pairs of the host
// experts in sorted order, for moe_expert_ffn on the device and the host
// kernel on the rest. All arrays in host memory.
extern "C" int moe_permute_split(const int32_t *offsets, const int32_t *sorted_pair, int E,
                                 const uint8_t *host_mask, int32_t *dev_offsets,
                                 int32_t *dev_sorted_pair, int32_t *host_pairs, int *n_host) {
    if (!offsets || E < 1 || !host_mask || !dev_offsets || !n_host) return MOE_EINVAL;
    const int n = offsets[E];
    if (n < 0 || offsets[0] != 0) return MOE_EINVAL;
    for (int e = 0; e < E; ++e)
        if (offsets[e + 1] < offsets[e]) return MOE_EINVAL;
    if (n > 0 && (!sorted_pair || !dev_sorted_pair || !host_pairs)) return MOE_EINVAL;
    int d = 0, h = 0;
    for (int e = 0; e < E; ++e) {
        dev_offsets[e] = d;
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
            if (host_mask[e]) host_pairs[h++] = sorted_pair[r];
            else dev_sorted_pair[d++] = sorted_pair[r];
        }
    }
    dev_offsets[E] = d;
    *n_host = h;
    return MOE_OK;
}
