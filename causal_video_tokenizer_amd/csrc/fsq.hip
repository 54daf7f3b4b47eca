// FSQ quantize / dequantize kernels.
//
// FSQ as described in "NVIDIA Cosmos Tokenizer 完全指南", section 7.2: each
// latent channel is bounded with tanh and rounded to its own level count,
// the digits form one mixed-radix index (codes_to_indices) and the index is
// turned back into codes without any codebook table (indices_to_codes).
//
// Quantize.  The bound tanh(z + s) h - o is strictly increasing in z, so the
// rounded value changes only where the bound crosses a half-integer.  Those
// breakpoints are computed once per call on the host in double precision and
// adjusted to the float32 grid (see fsq_params in abi.cpp), so that
// "z >= thr" holds exactly when z lies above the breakpoint.  The digit is
// then the number of breakpoints at or below z: no transcendental is evaluated
// per element and the decision equals the exact one for every float input
// not within double rounding of a breakpoint.
//
// Mapping: one thread per run of 8 consecutive positions.  Planar (NCTHW)
// latents are read as one 16-byte (bf16) or two 16-byte (fp32) streaming loads per
// channel; NTHWC latents as the thread's contiguous 8*D-element span.  Indices
// are written as two 16-byte stores.  Ragged tails and plane sizes that are not
// multiples of 8 take the per-position path.
#include <math.h>

#include "cvt_internal.h"

namespace cvt {
namespace {

constexpr int G = 8;  // positions per thread

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
    const uint4 u = ld_stream16(p);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
    const uint4 a = ld_stream16(p);
    const uint4 b = ld_stream16(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ float ld1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ void st1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void st1(float* p, float v) { *p = v; }

// Level-set descriptors.  Runtime<D>: everything read from FsqParams.  Default:
// the levels (8,8,8,5,5,5) of the pages, with compile-time breakpoint counts,
// place values and power-of-two code scales (thresholds stay runtime values).
struct RuntimeLevels {};
struct DefaultLevels {
    static constexpr int D = 6;
    __device__ static constexpr int L(int i) { return i < 3 ? 8 : 5; }
    __device__ static constexpr int nthr(int i) { return L(i) - 1; }
    __device__ static constexpr int half(int i) { return L(i) / 2; }
    __device__ static constexpr float inv_half(int i) { return i < 3 ? 0.25f : 0.5f; }
    __device__ static constexpr int basis(int i) {
        return i == 0 ? 1 : i == 1 ? 8 : i == 2 ? 64 : i == 3 ? 512 : i == 4 ? 2560 : 12800;
    }
    static constexpr int codebook = 64000;
};

template <int NT>
__device__ __forceinline__ int digit_exact(float v, const float* thr) {
    int d = 0;
#pragma unroll
    for (int j = 0; j < NT; ++j) d += (v >= thr[j]) ? 1 : 0;
    return d;
}

// NaN for a NaN input, else +0: added to a code it marks NaN latents without a branch
// (+-inf inputs keep their saturated codes).
__device__ __forceinline__ float nan_or_zero(float x) { return (x != x) ? __builtin_nanf("") : 0.0f; }

// Digit of channel i under the default levels (i is a constant after unrolling).
__device__ __forceinline__ int digit_default(int i, float x, const FsqParams& p) {
    return i < 3 ? digit_exact<7>(x, p.thr[i]) : digit_exact<4>(x, p.thr[i]);
}

template <int NT>
__device__ __forceinline__ int digit_of(float v, const float* thr) {
    int d = 0;
#pragma unroll
    for (int j = 0; j < NT; ++j) d += (v >= thr[j]) ? 1 : 0;  // padded entries are NaN: never counted
    return d;
}

__device__ __forceinline__ float code_of(int d, int half) {
    return (float)(d - half) / (float)half;
}

// Quantize with the default levels: 8 positions per thread, compile-time
// breakpoint counts (7 for L = 8, 4 for L = 5); codes only when CODES.
template <typename T, int LAYOUT, bool CODES>
__global__ __launch_bounds__(256) void fsq_quantize_default_kernel(const T* __restrict__ z, int32_t* __restrict__ idx,
                                                                   T* __restrict__ codes, FsqParams p, long long npb,
                                                                   long long total) {
    using LV = DefaultLevels;
    constexpr int D = LV::D;
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long pos0 = g * G;
    if (pos0 >= total) return;
    int acc[G];
    bool nan_[G];
#pragma unroll
    for (int k = 0; k < G; ++k) { acc[k] = 0; nan_[k] = false; }
    if (pos0 + G <= total) {
        if (LAYOUT == CVT_NCTHW) {
            const long long b = pos0 / npb, r = pos0 - b * npb;
            float v[D][G];
#pragma unroll
            for (int i = 0; i < D; ++i) load8<T>(z + ((size_t)b * D + i) * npb + r, v[i]);
#pragma unroll
            for (int i = 0; i < D; ++i) {
                float cv[G];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    const int d = digit_default(i, v[i][k], p);
                    acc[k] += d * LV::basis(i);
                    nan_[k] |= (v[i][k] != v[i][k]);
                    if (CODES) cv[k] = (float)(d - LV::half(i)) * LV::inv_half(i) + nan_or_zero(v[i][k]);
                }
                if (CODES) store8(codes + ((size_t)b * D + i) * npb + r, cv);
            }
        } else {
            float v[D][G];  // D chunks of 8 consecutive elements = 8 positions x 6 channels
#pragma unroll
            for (int c8 = 0; c8 < D; ++c8) load8<T>(z + (size_t)pos0 * D + c8 * G, v[c8]);
#pragma unroll
            for (int c8 = 0; c8 < D; ++c8) {
                float cv[G];
#pragma unroll
                for (int e = 0; e < G; ++e) {
                    const int flat = c8 * G + e, k = flat / D, i = flat % D;
                    const float x = v[c8][e];
                    const int d = digit_default(i, x, p);
                    acc[k] += d * LV::basis(i);
                    nan_[k] |= (x != x);
                    if (CODES) cv[e] = (float)(d - LV::half(i)) * LV::inv_half(i) + nan_or_zero(x);
                }
                if (CODES) store8(codes + (size_t)pos0 * D + c8 * G, cv);
            }
        }
        int4 o0, o1;
        o0.x = nan_[0] ? -1 : acc[0]; o0.y = nan_[1] ? -1 : acc[1];
        o0.z = nan_[2] ? -1 : acc[2]; o0.w = nan_[3] ? -1 : acc[3];
        o1.x = nan_[4] ? -1 : acc[4]; o1.y = nan_[5] ? -1 : acc[5];
        o1.z = nan_[6] ? -1 : acc[6]; o1.w = nan_[7] ? -1 : acc[7];
        *reinterpret_cast<int4*>(idx + pos0) = o0;
        *reinterpret_cast<int4*>(idx + pos0 + 4) = o1;
        return;
    }
    for (long long pos = pos0; pos < total; ++pos) {  // ragged tail (< 8 positions)
        int a = 0;
        bool isnan_ = false;
        const long long b = pos / npb, r = pos - b * npb;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const size_t off = LAYOUT == CVT_NCTHW ? ((size_t)b * D + i) * npb + r : (size_t)pos * D + i;
            const float x = ld1(z + off);
            const int d = digit_exact<7>(x, p.thr[i]);  // unused breakpoints are NaN
            a += d * LV::basis(i);
            isnan_ |= (x != x);
            if (CODES) st1(codes + off, (x != x) ? __builtin_nanf("") : (float)(d - LV::half(i)) * LV::inv_half(i));
        }
        idx[pos] = isnan_ ? -1 : a;
    }
}

// DC: compile-time D (0 = runtime); NT: breakpoints per channel (padded).
template <typename T, int LAYOUT, int DC, int NT>
__global__ __launch_bounds__(256) void fsq_quantize_kernel(const T* __restrict__ z, int32_t* __restrict__ idx,
                                                           T* __restrict__ codes, FsqParams p,
                                                           long long npb, long long total, int vec) {
    const int D = DC > 0 ? DC : p.D;
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long pos0 = g * G;
    if (pos0 >= total) return;

    if (vec && pos0 + G <= total) {
        int acc[G];
        bool nan_[G];
#pragma unroll
        for (int k = 0; k < G; ++k) { acc[k] = 0; nan_[k] = false; }
        if (LAYOUT == CVT_NCTHW) {
            const long long b = pos0 / npb, r = pos0 - b * npb;
#pragma unroll
            for (int i = 0; i < (DC > 0 ? DC : FSQ_MAX_D); ++i) {
                if (DC == 0 && i >= D) break;
                float v[G];
                load8<T>(z + ((size_t)b * D + i) * npb + r, v);
                float cv[G];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    const int d = digit_of<NT>(v[k], p.thr[i]);
                    acc[k] += d * p.basis[i];
                    nan_[k] |= (v[k] != v[k]);
                    cv[k] = (v[k] != v[k]) ? __builtin_nanf("") : code_of(d, p.half[i]);
                }
                if (codes) store8(codes + ((size_t)b * D + i) * npb + r, cv);
            }
        } else {
            const T* src = z + (size_t)pos0 * D;
            T* dst = codes ? codes + (size_t)pos0 * D : nullptr;
#pragma unroll
            for (int c8 = 0; c8 < (DC > 0 ? DC : FSQ_MAX_D); ++c8) {  // D chunks of 8 elements
                if (DC == 0 && c8 >= D) break;
                float v[G], cv[G];
                load8<T>(src + c8 * G, v);
#pragma unroll
                for (int e = 0; e < G; ++e) {
                    const int flat = c8 * G + e;  // = k * D + i
                    const int k = flat / D, i = flat - (flat / D) * D;
                    const int d = digit_of<NT>(v[e], p.thr[i]);
                    acc[k] += d * p.basis[i];
                    nan_[k] |= (v[e] != v[e]);
                    cv[e] = (v[e] != v[e]) ? __builtin_nanf("") : code_of(d, p.half[i]);
                }
                if (dst) store8(dst + c8 * G, cv);
            }
        }
        int4 o0, o1;
        o0.x = nan_[0] ? -1 : acc[0]; o0.y = nan_[1] ? -1 : acc[1];
        o0.z = nan_[2] ? -1 : acc[2]; o0.w = nan_[3] ? -1 : acc[3];
        o1.x = nan_[4] ? -1 : acc[4]; o1.y = nan_[5] ? -1 : acc[5];
        o1.z = nan_[6] ? -1 : acc[6]; o1.w = nan_[7] ? -1 : acc[7];
        *reinterpret_cast<int4*>(idx + pos0) = o0;
        *reinterpret_cast<int4*>(idx + pos0 + 4) = o1;
        return;
    }

    // per-position path (tails, unaligned planes)
    for (long long pos = pos0; pos < pos0 + G && pos < total; ++pos) {
        int acc = 0;
        bool isnan_ = false;
        const long long b = pos / npb, r = pos - b * npb;
        for (int i = 0; i < D; ++i) {
            const size_t off = LAYOUT == CVT_NCTHW ? ((size_t)b * D + i) * npb + r : (size_t)pos * D + i;
            const float v = ld1(z + off);
            const int d = digit_of<NT>(v, p.thr[i]);
            acc += d * p.basis[i];
            isnan_ |= (v != v);
            if (codes) st1(codes + off, (v != v) ? __builtin_nanf("") : code_of(d, p.half[i]));
        }
        idx[pos] = isnan_ ? -1 : acc;
    }
}

// Exact floor(n / L) for 0 <= n < 2^31 and 2 <= L <= 16.  With l = ceil(log2 L),
// M = ceil(2^(31+l) / L) < 2^32 and n M / 2^(31+l) exceeds n / L by less than
// n / 2^(31+l) < 2^-l <= 1/L, the smallest gap between n / L and the next
// integer, so floor(mulhi(n, M) / 2^(l-1)) = floor(n / L).
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t M, int sh) {
    return __umulhi(n, M) >> sh;
}

// Dequantize with the default levels: compile-time radices (the compiler
// divides by 8 and 5 with shifts / multiply-high) and power-of-two code scales.
template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void fsq_dequantize_default_kernel(const int32_t* __restrict__ idx,
                                                                     T* __restrict__ codes, long long npb,
                                                                     long long total, int32_t* __restrict__ invalid) {
    using LV = DefaultLevels;
    constexpr int D = LV::D;
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long pos0 = g * G;
    if (pos0 >= total) return;
    int nbad = 0;
    if (pos0 + G <= total) {
        const uint4 ua = ld_stream16(idx + pos0), uc = ld_stream16(idx + pos0 + 4);
        const int4 a = make_int4((int)ua.x, (int)ua.y, (int)ua.z, (int)ua.w);
        const int4 c = make_int4((int)uc.x, (int)uc.y, (int)uc.z, (int)uc.w);
        const int id[G] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        float cv[D][G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const bool bad = (unsigned)id[k] >= (unsigned)LV::codebook;
            nbad += bad ? 1 : 0;
            // branchless invalid handling: the digits of 0 plus a NaN addend
            const float nan_add = bad ? __builtin_nanf("") : 0.0f;
            uint32_t rem = bad ? 0u : (uint32_t)id[k];
#pragma unroll
            for (int i = 0; i < D; ++i) {
                const uint32_t q = rem / (uint32_t)LV::L(i);
                const int d = (int)(rem - q * (uint32_t)LV::L(i));
                rem = q;
                cv[i][k] = (float)(d - LV::half(i)) * LV::inv_half(i) + nan_add;
            }
        }
        if (LAYOUT == CVT_NCTHW) {
            const long long b = pos0 / npb, r = pos0 - b * npb;
#pragma unroll
            for (int i = 0; i < D; ++i) store8(codes + ((size_t)b * D + i) * npb + r, cv[i]);
        } else {
            float flat[G * D];
#pragma unroll
            for (int k = 0; k < G; ++k)
#pragma unroll
                for (int i = 0; i < D; ++i) flat[k * D + i] = cv[i][k];
#pragma unroll
            for (int c8 = 0; c8 < D; ++c8) store8(codes + (size_t)pos0 * D + c8 * G, flat + c8 * G);
        }
    } else {
        for (long long pos = pos0; pos < total; ++pos) {
            const int v = idx[pos];
            const bool bad = (unsigned)v >= (unsigned)LV::codebook;
            nbad += bad ? 1 : 0;
            uint32_t rem = bad ? 0u : (uint32_t)v;
            const long long b = pos / npb, r = pos - b * npb;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                const uint32_t q = rem / (uint32_t)LV::L(i);
                const int d = (int)(rem - q * (uint32_t)LV::L(i));
                rem = q;
                const size_t off = LAYOUT == CVT_NCTHW ? ((size_t)b * D + i) * npb + r : (size_t)pos * D + i;
                st1(codes + off, bad ? __builtin_nanf("") : (float)(d - LV::half(i)) * LV::inv_half(i));
            }
        }
    }
    if (invalid && nbad) atomicAdd(invalid, nbad);
}

// Dequantize with the default levels through two LDS tables.  With radices
// (8,8,8,5,5,5) the index splits into lo = idx mod 512 (the three base-8 digits) and
// hi = idx / 512 < 125 (the three base-5 digits); each table row holds the three
// codes of its digits, packed as the output type (bf16 pairs or floats), and row
// 512 / 125 holds NaNs for invalid indices.  Per position this is two LDS reads and
// a few byte permutes instead of six divisions and conversions.  Each workgroup
// fills its tables once and then walks several 8-position groups.
template <typename T>
struct CodeRow;
template <>
struct CodeRow<uint16_t> {
    using type = uint2;  // x = c0 | c1 << 16, y = c2
    __device__ static type make(float c0, float c1, float c2) {
        return make_uint2(pack_bf16x2(c0, c1), pack_bf16x2(c2, 0.0f));
    }
};
template <>
struct CodeRow<float> {
    using type = float4;
    __device__ static type make(float c0, float c1, float c2) { return make_float4(c0, c1, c2, 0.0f); }
};

constexpr int DQ_GROUPS = 4;  // 8-position groups per thread

template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void fsq_dequantize_lut_kernel(const int32_t* __restrict__ idx, T* __restrict__ codes,
                                                                 long long npb, long long total,
                                                                 int32_t* __restrict__ invalid) {
    using Row = typename CodeRow<T>::type;
    __shared__ Row lutA[513];
    __shared__ Row lutB[126];
    const float qnan = __builtin_nanf("");
    for (int e = threadIdx.x; e < 513 + 126; e += blockDim.x) {
        if (e < 512) {
            lutA[e] = CodeRow<T>::make(((e & 7) - 4) * 0.25f, (((e >> 3) & 7) - 4) * 0.25f, ((e >> 6) - 4) * 0.25f);
        } else if (e == 512) {
            lutA[e] = CodeRow<T>::make(qnan, qnan, qnan);
        } else {
            const int h = e - 513;
            lutB[h] = h < 125 ? CodeRow<T>::make((h % 5 - 2) * 0.5f, ((h / 5) % 5 - 2) * 0.5f, (h / 25 - 2) * 0.5f)
                              : CodeRow<T>::make(qnan, qnan, qnan);
        }
    }
    __syncthreads();

    int nbad = 0;
    for (int r = 0; r < DQ_GROUPS; ++r) {
        const long long pos0 = ((long long)(blockIdx.x * DQ_GROUPS + r) * blockDim.x + threadIdx.x) * G;
        if (pos0 >= total) break;
        if (pos0 + G <= total) {
            const uint4 ua = ld_stream16(idx + pos0), uc = ld_stream16(idx + pos0 + 4);
            const uint32_t id[G] = {ua.x, ua.y, ua.z, ua.w, uc.x, uc.y, uc.z, uc.w};
            Row A[G], Bv[G];
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const bool bad = id[k] >= 64000u;
                nbad += bad ? 1 : 0;
                A[k] = lutA[bad ? 512 : (id[k] & 511u)];
                Bv[k] = lutB[bad ? 125 : (id[k] >> 9)];
            }
            if constexpr (sizeof(T) == 2) {
                // bf16: combine 16-bit fields with byte permutes
                auto lo2 = [](uint32_t p, uint32_t q) { return __builtin_amdgcn_perm(q, p, 0x05040100u); };
                auto hi2 = [](uint32_t p, uint32_t q) { return __builtin_amdgcn_perm(q, p, 0x07060302u); };
                if (LAYOUT == CVT_NCTHW) {
                    const long long b = pos0 / npb, rr = pos0 - b * npb;
                    uint4 o[6];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int p = 2 * j, q = 2 * j + 1;
                        (&o[0].x)[j] = lo2(A[p].x, A[q].x);
                        (&o[1].x)[j] = hi2(A[p].x, A[q].x);
                        (&o[2].x)[j] = lo2(A[p].y, A[q].y);
                        (&o[3].x)[j] = lo2(Bv[p].x, Bv[q].x);
                        (&o[4].x)[j] = hi2(Bv[p].x, Bv[q].x);
                        (&o[5].x)[j] = lo2(Bv[p].y, Bv[q].y);
                    }
#pragma unroll
                    for (int i = 0; i < 6; ++i)
                        *reinterpret_cast<uint4*>(codes + ((size_t)b * 6 + i) * npb + rr) = o[i];
                } else {
                    // per position: (c0 c1) (c2 c3) (c4 c5)
                    uint32_t w[3 * G];
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        w[3 * k] = A[k].x;
                        w[3 * k + 1] = lo2(A[k].y, Bv[k].x);
                        w[3 * k + 2] = __builtin_amdgcn_perm(Bv[k].y, Bv[k].x, 0x05040302u);
                    }
                    uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)pos0 * 6);
#pragma unroll
                    for (int c = 0; c < 6; ++c) dst[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
                }
            } else {
                float cv[6][G];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    cv[0][k] = A[k].x; cv[1][k] = A[k].y; cv[2][k] = A[k].z;
                    cv[3][k] = Bv[k].x; cv[4][k] = Bv[k].y; cv[5][k] = Bv[k].z;
                }
                if (LAYOUT == CVT_NCTHW) {
                    const long long b = pos0 / npb, rr = pos0 - b * npb;
#pragma unroll
                    for (int i = 0; i < 6; ++i) store8(codes + ((size_t)b * 6 + i) * npb + rr, cv[i]);
                } else {
                    float flat[6 * G];
#pragma unroll
                    for (int k = 0; k < G; ++k)
#pragma unroll
                        for (int i = 0; i < 6; ++i) flat[k * 6 + i] = cv[i][k];
#pragma unroll
                    for (int c8 = 0; c8 < 6; ++c8) store8(codes + (size_t)pos0 * 6 + c8 * G, flat + c8 * G);
                }
            }
        } else {
            for (long long pos = pos0; pos < total; ++pos) {  // ragged tail (< 8 positions)
                const uint32_t v = (uint32_t)idx[pos];
                const bool bad = v >= 64000u;
                nbad += bad ? 1 : 0;
                uint32_t rem = bad ? 0u : v;
                const long long b = pos / npb, rr = pos - b * npb;
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    const uint32_t L = i < 3 ? 8u : 5u;
                    const uint32_t q = rem / L;
                    const int d = (int)(rem - q * L);
                    rem = q;
                    const float c = bad ? qnan : (float)(d - (int)(L / 2)) * (i < 3 ? 0.25f : 0.5f);
                    const size_t off = LAYOUT == CVT_NCTHW ? ((size_t)b * 6 + i) * npb + rr : (size_t)pos * 6 + i;
                    st1(codes + off, c);
                }
            }
        }
    }
    if (invalid && nbad) atomicAdd(invalid, nbad);
}

template <typename T, int LAYOUT, int DC>
__global__ __launch_bounds__(256) void fsq_dequantize_kernel(const int32_t* __restrict__ idx, T* __restrict__ codes,
                                                             FsqParams p, long long npb, long long total,
                                                             int vec, int32_t* __restrict__ invalid) {
    const int D = DC > 0 ? DC : p.D;
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long pos0 = g * G;
    if (pos0 >= total) return;
    int nbad = 0;


    if (vec && pos0 + G <= total) {
        const uint4 ua = ld_stream16(idx + pos0), uc = ld_stream16(idx + pos0 + 4);
        const int4 a = make_int4((int)ua.x, (int)ua.y, (int)ua.z, (int)ua.w);
        const int4 c = make_int4((int)uc.x, (int)uc.y, (int)uc.z, (int)uc.w);
        const int id[G] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        bool bad[G];
        uint32_t rem[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            bad[k] = id[k] < 0 || id[k] >= p.codebook;
            nbad += bad[k] ? 1 : 0;
            rem[k] = bad[k] ? 0u : (uint32_t)id[k];
        }
        if (LAYOUT == CVT_NCTHW) {
            const long long b = pos0 / npb, r = pos0 - b * npb;
#pragma unroll
            for (int i = 0; i < (DC > 0 ? DC : FSQ_MAX_D); ++i) {
                if (DC == 0 && i >= D) break;
                float cv[G];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    const uint32_t q = div_magic(rem[k], p.magic[i], p.shift[i]);
                    const int d = (int)(rem[k] - q * (uint32_t)p.levels[i]);
                    rem[k] = q;
                    cv[k] = bad[k] ? __builtin_nanf("") : code_of(d, p.half[i]);
                }
                store8(codes + ((size_t)b * D + i) * npb + r, cv);
            }
        } else {
            T* dst = codes + (size_t)pos0 * D;
            float cv[G * FSQ_MAX_D];
#pragma unroll
            for (int k = 0; k < G; ++k)
#pragma unroll
                for (int i = 0; i < (DC > 0 ? DC : FSQ_MAX_D); ++i) {
                    if (DC == 0 && i >= D) break;
                    const uint32_t q = div_magic(rem[k], p.magic[i], p.shift[i]);
                    const int d = (int)(rem[k] - q * (uint32_t)p.levels[i]);
                    rem[k] = q;
                    cv[k * D + i] = bad[k] ? __builtin_nanf("") : code_of(d, p.half[i]);
                }
#pragma unroll
            for (int c8 = 0; c8 < (DC > 0 ? DC : FSQ_MAX_D); ++c8) {
                if (DC == 0 && c8 >= D) break;
                store8(dst + c8 * G, cv + c8 * G);
            }
        }
    } else {
        for (long long pos = pos0; pos < pos0 + G && pos < total; ++pos) {
            const int v = idx[pos];
            const bool bd = v < 0 || v >= p.codebook;
            nbad += bd ? 1 : 0;
            uint32_t rem = bd ? 0u : (uint32_t)v;
            const long long b = pos / npb, r = pos - b * npb;
            for (int i = 0; i < D; ++i) {
                const uint32_t q = div_magic(rem, p.magic[i], p.shift[i]);
                const int d = (int)(rem - q * (uint32_t)p.levels[i]);
                rem = q;
                const size_t off = LAYOUT == CVT_NCTHW ? ((size_t)b * D + i) * npb + r : (size_t)pos * D + i;
                st1(codes + off, bd ? __builtin_nanf("") : code_of(d, p.half[i]));
            }
        }
    }
    if (invalid && nbad) atomicAdd(invalid, nbad);
}

bool is_default(const FsqParams& p) {
    static const int def[6] = {8, 8, 8, 5, 5, 5};
    if (p.D != 6) return false;
    for (int i = 0; i < 6; ++i)
        if (p.levels[i] != def[i]) return false;
    return true;
}

template <typename T, int LAYOUT, int DC>
hipError_t quantize_nt(const void* z, int32_t* idx, void* codes, const FsqParams& p, long long npb,
                       long long total, int vec, hipStream_t s) {
    int maxthr = 0;
    for (int i = 0; i < p.D; ++i) maxthr = p.nthr[i] > maxthr ? p.nthr[i] : maxthr;
    const long long nthreads = (total + G - 1) / G;
    const long long nblk = (nthreads + 255) / 256;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblk), block(256);
#define CVT_FSQ_Q(NT) \
    hipLaunchKernelGGL((fsq_quantize_kernel<T, LAYOUT, DC, NT>), grid, block, 0, s, (const T*)z, idx, (T*)codes, p, npb, total, vec)
    if (maxthr <= 1) CVT_FSQ_Q(1);
    else if (maxthr <= 3) CVT_FSQ_Q(3);
    else if (maxthr <= 4) CVT_FSQ_Q(4);
    else if (maxthr <= 7) CVT_FSQ_Q(7);
    else CVT_FSQ_Q(15);
#undef CVT_FSQ_Q
    return hipGetLastError();
}

template <typename T, int LAYOUT>
hipError_t quantize_t(const void* z, int32_t* idx, void* codes, const FsqParams& p, long long B, long long npb,
                      hipStream_t s) {
    const long long total = B * npb;
    // vector path: 8-aligned plane starts for NCTHW; NTHWC spans are always contiguous
    const int vec = LAYOUT == CVT_NTHWC ? 1 : (npb % G == 0);
    if (is_default(p) && vec) {
        const long long nblk = ((total + G - 1) / G + 255) / 256;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        if (codes)
            hipLaunchKernelGGL((fsq_quantize_default_kernel<T, LAYOUT, true>), dim3((unsigned)nblk), dim3(256), 0, s,
                               (const T*)z, idx, (T*)codes, p, npb, total);
        else
            hipLaunchKernelGGL((fsq_quantize_default_kernel<T, LAYOUT, false>), dim3((unsigned)nblk), dim3(256), 0, s,
                               (const T*)z, idx, (T*)nullptr, p, npb, total);
        return hipGetLastError();
    }
    if (p.D == 6) return quantize_nt<T, LAYOUT, 6>(z, idx, codes, p, npb, total, vec, s);
    return quantize_nt<T, LAYOUT, 0>(z, idx, codes, p, npb, total, vec, s);
}

template <typename T, int LAYOUT>
hipError_t dequantize_t(const int32_t* idx, void* codes, const FsqParams& p, long long B, long long npb,
                        int32_t* invalid, hipStream_t s) {
    const long long total = B * npb;
    const int vec = LAYOUT == CVT_NTHWC ? 1 : (npb % G == 0);
    const long long nthreads = (total + G - 1) / G;
    const long long nblk = (nthreads + 255) / 256;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (is_default(p) && vec)
        hipLaunchKernelGGL((fsq_dequantize_lut_kernel<T, LAYOUT>), dim3((unsigned)((nblk + DQ_GROUPS - 1) / DQ_GROUPS)),
                           dim3(256), 0, s, idx, (T*)codes, npb, total, invalid);
    else if (p.D == 6)
        hipLaunchKernelGGL((fsq_dequantize_kernel<T, LAYOUT, 6>), dim3((unsigned)nblk), dim3(256), 0, s, idx, (T*)codes, p,
                           npb, total, vec, invalid);
    else
        hipLaunchKernelGGL((fsq_dequantize_kernel<T, LAYOUT, 0>), dim3((unsigned)nblk), dim3(256), 0, s, idx, (T*)codes, p,
                           npb, total, vec, invalid);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fsq_quantize(const void* z, int z_dtype, int z_layout, int32_t* idx, void* codes,
                               const FsqParams& p, long long B, long long npb, hipStream_t s) {
    if (z_dtype == CVT_BF16)
        return z_layout == CVT_NTHWC ? quantize_t<uint16_t, CVT_NTHWC>(z, idx, codes, p, B, npb, s)
                                     : quantize_t<uint16_t, CVT_NCTHW>(z, idx, codes, p, B, npb, s);
    return z_layout == CVT_NTHWC ? quantize_t<float, CVT_NTHWC>(z, idx, codes, p, B, npb, s)
                                 : quantize_t<float, CVT_NCTHW>(z, idx, codes, p, B, npb, s);
}

hipError_t launch_fsq_dequantize(const int32_t* idx, void* codes, int c_dtype, int c_layout, const FsqParams& p,
                                 long long B, long long npb, int32_t* invalid, hipStream_t s) {
    if (c_dtype == CVT_BF16)
        return c_layout == CVT_NTHWC ? dequantize_t<uint16_t, CVT_NTHWC>(idx, codes, p, B, npb, invalid, s)
                                     : dequantize_t<uint16_t, CVT_NCTHW>(idx, codes, p, B, npb, invalid, s);
    return c_layout == CVT_NTHWC ? dequantize_t<float, CVT_NTHWC>(idx, codes, p, B, npb, invalid, s)
                                 : dequantize_t<float, CVT_NCTHW>(idx, codes, p, B, npb, invalid, s);
}

}  // namespace cvt
