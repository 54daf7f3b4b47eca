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
// channel; NTHWC latents as the thread's contiguous 8*D-element span.  For the
// default levels each wave takes 512 positions and moves NTHWC spans and index runs
// through LDS, so every wave-wide access is one contiguous 1 KB (see "Wave tiles").
// Ragged tails and plane sizes that are not multiples of 8 take the per-position path.
#include <math.h>

#include <algorithm>

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

// Wave tiles.  The default-level kernels give each wave 512 consecutive positions (8 per
// lane).  Data that is contiguous per lane but interleaved across lanes - an NTHWC span
// of 8 positions x D channels, or 8 indices - is moved through a wave-private LDS tile,
// so that every global load or store instruction of the wave covers one contiguous
// 1 KB (lane l at bytes 16 l) instead of 64 strided pieces.  A wave reads back only what
// it wrote and its LDS accesses execute in order, so no barrier is needed.
constexpr int WAVE_POS = 64 * G;

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16-byte chunk <-> 8 bf16 or 4 float values
__device__ __forceinline__ void unpack16(const uint4 u, float* v, uint16_t) {
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void unpack16(const uint4 u, float* v, float) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y); v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ uint4 pack16(const float* v, uint16_t) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ uint4 pack16(const float* v, float) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}

// Quantize with the default levels: compile-time breakpoint counts (7 for L = 8, 4 for
// L = 5); codes only when CODES.  Full wave tiles take the staged path; the positions
// after the last full tile (fewer than 512) are done by one more wave, 8 per lane, with
// direct accesses and a per-position path for the last partial group.
template <typename T, int LAYOUT, bool CODES>
__global__ __launch_bounds__(256) void fsq_quantize_default_kernel(const T* __restrict__ z, int32_t* __restrict__ idx,
                                                                   T* __restrict__ codes, FsqParams p, long long npb,
                                                                   long long total) {
    using LV = DefaultLevels;
    constexpr int D = LV::D;
    constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    constexpr int NCH = G * D / EPC;          // chunks of one lane's NTHWC span (6 bf16, 12 fp32)
    constexpr int SCH = LAYOUT == CVT_NTHWC ? NCH : 2;  // staged chunks per lane (NCTHW: indices only)
    __shared__ uint4 stage[4][64 * SCH];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint4* st = stage[w];
    // Planar latents: grid row blockIdx.y is one clip (its npb positions, a multiple of 8
    // on this path), so the plane offsets need no division; NTHWC: one row over all.
    const long long base = LAYOUT == CVT_NCTHW ? (long long)blockIdx.y * npb : 0;
    const long long span = LAYOUT == CVT_NCTHW ? npb : total;
    const long long wave_id = (long long)blockIdx.x * 4 + w;  // wave tile within the row
    const long long nfull = span / WAVE_POS;
    if (wave_id > nfull) return;
    const bool full = wave_id < nfull;
    const long long lpos0 = wave_id * WAVE_POS + lane * G;
    if (!full && lpos0 >= span) return;
    const long long pos0 = base + lpos0;

    if (full || lpos0 + G <= span) {
        float v[D][G];  // v[i][k]: channel i of position pos0 + k
        long long b = 0, r = 0;
        if (LAYOUT == CVT_NCTHW) {
            b = blockIdx.y;
            r = lpos0;
#pragma unroll
            for (int i = 0; i < D; ++i) load8<T>(z + ((size_t)b * D + i) * npb + r, v[i]);
        } else {
            float flat[G * D];
            if (full) {
                const uint4* src = reinterpret_cast<const uint4*>(z + (size_t)(wave_id * WAVE_POS) * D);
                uint4 t[NCH];
#pragma unroll
                for (int c = 0; c < NCH; ++c) t[c] = ld_stream16(src + c * 64 + lane);
#pragma unroll
                for (int c = 0; c < NCH; ++c) st[c * 64 + lane] = t[c];
                wave_lds_sync();
#pragma unroll
                for (int c = 0; c < NCH; ++c) unpack16(st[lane * NCH + c], flat + c * EPC, T());
                wave_lds_sync();
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(z + (size_t)pos0 * D);
#pragma unroll
                for (int c = 0; c < NCH; ++c) unpack16(ld_stream16(src + c), flat + c * EPC, T());
            }
#pragma unroll
            for (int k = 0; k < G; ++k)
#pragma unroll
                for (int i = 0; i < D; ++i) v[i][k] = flat[k * D + i];
        }

        int acc[G];
        bool nan_[G];
        float cv[D][G];
#pragma unroll
        for (int k = 0; k < G; ++k) { acc[k] = 0; nan_[k] = false; }
#pragma unroll
        for (int i = 0; i < D; ++i)
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const float x = v[i][k];
                const int d = digit_default(i, x, p);
                acc[k] += d * LV::basis(i);
                nan_[k] |= (x != x);
                if (CODES) cv[i][k] = (float)(d - LV::half(i)) * LV::inv_half(i) + nan_or_zero(x);
            }

        if (CODES) {
            if (LAYOUT == CVT_NCTHW) {
#pragma unroll
                for (int i = 0; i < D; ++i) store8(codes + ((size_t)b * D + i) * npb + r, cv[i]);
            } else {
                float flat[G * D];
#pragma unroll
                for (int k = 0; k < G; ++k)
#pragma unroll
                    for (int i = 0; i < D; ++i) flat[k * D + i] = cv[i][k];
                if (full) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c) st[lane * NCH + c] = pack16(flat + c * EPC, T());
                    wave_lds_sync();
                    uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)(wave_id * WAVE_POS) * D);
#pragma unroll
                    for (int c = 0; c < NCH; ++c) st_stream16(dst + c * 64 + lane, st[c * 64 + lane]);
                    wave_lds_sync();
                } else {
                    uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)pos0 * D);
#pragma unroll
                    for (int c = 0; c < NCH; ++c) dst[c] = pack16(flat + c * EPC, T());
                }
            }
        }

        int4 o0, o1;
        o0.x = nan_[0] ? -1 : acc[0]; o0.y = nan_[1] ? -1 : acc[1];
        o0.z = nan_[2] ? -1 : acc[2]; o0.w = nan_[3] ? -1 : acc[3];
        o1.x = nan_[4] ? -1 : acc[4]; o1.y = nan_[5] ? -1 : acc[5];
        o1.z = nan_[6] ? -1 : acc[6]; o1.w = nan_[7] ? -1 : acc[7];
        if (full) {
            st[2 * lane] = *reinterpret_cast<uint4*>(&o0);
            st[2 * lane + 1] = *reinterpret_cast<uint4*>(&o1);
            wave_lds_sync();
            uint4* dst = reinterpret_cast<uint4*>(idx + base + wave_id * WAVE_POS);
            st_stream16(dst + lane, st[lane]);
            st_stream16(dst + 64 + lane, st[64 + lane]);
        } else {
            *reinterpret_cast<int4*>(idx + pos0) = o0;
            *reinterpret_cast<int4*>(idx + pos0 + 4) = o1;
        }
        return;
    }
    for (long long pos = pos0; pos < base + span; ++pos) {  // last partial group (< 8 positions, NTHWC only)
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


// Dequantize with the default levels.  With radices (8,8,8,5,5,5) the index splits into
// lo = idx mod 512, whose three octal digits are bit fields, and hi = idx / 512 < 125,
// whose base-5 digits come from two exact multiply-shift divisions (hi / 5 =
// (hi * 52429) >> 18 and hi / 25 = (hi * 5243) >> 17 for hi < 125).  Codes are
// (d - L/2) * (2/L) with power-of-two scales, exact in bf16 and fp32; invalid indices
// add a NaN.  Each wave takes one 512-position tile (see "Wave tiles").
template <typename T>
struct CodeRow;
template <>
struct CodeRow<uint16_t> {
    using type = uint2;  // three codes: x = c0 | c1 << 16, y = c2
    __device__ static type make(float c0, float c1, float c2) {
        return make_uint2(pack_bf16x2(c0, c1), pack_bf16x2(c2, 0.0f));
    }
};
template <>
struct CodeRow<float> {
    using type = float4;
    __device__ static type make(float c0, float c1, float c2) { return make_float4(c0, c1, c2, 0.0f); }
};

template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void fsq_dequantize_default_kernel(const int32_t* __restrict__ idx, T* __restrict__ codes,
                                                                 long long npb, long long total,
                                                                 int32_t* __restrict__ invalid) {
    using Row = typename CodeRow<T>::type;
    constexpr int D = 6;
    constexpr int EPC = 16 / (int)sizeof(T);
    constexpr int NCH = G * D / EPC;  // chunks of one lane's NTHWC span (6 bf16, 12 fp32)
    constexpr int SCH = LAYOUT == CVT_NTHWC ? NCH : 2;  // staged chunks per lane (NCTHW: indices only)
    __shared__ uint4 stage[4][64 * SCH];
    const float qnan = __builtin_nanf("");

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint4* st = stage[w];
    const long long nfull = total / WAVE_POS;
    int nbad = 0;
    // grid-stride over the wave tiles (the launch covers all of them, one per wave)
    for (long long wave_id = (long long)blockIdx.x * 4 + w; wave_id <= nfull; wave_id += (long long)gridDim.x * 4) {
        const bool full = wave_id < nfull;
        const long long pos0 = wave_id * WAVE_POS + lane * G;
        if (!full && pos0 >= total) break;
        if (full || pos0 + G <= total) {
            uint4 ua, uc;
            if (full) {  // the wave's 512 indices as two contiguous 1 KB loads
                const uint4* src = reinterpret_cast<const uint4*>(idx + wave_id * WAVE_POS);
                const uint4 t0 = ld_stream16(src + lane), t1 = ld_stream16(src + 64 + lane);
                st[lane] = t0;
                st[64 + lane] = t1;
                wave_lds_sync();
                ua = st[2 * lane];
                uc = st[2 * lane + 1];
                wave_lds_sync();
            } else {
                ua = ld_stream16(idx + pos0);
                uc = ld_stream16(idx + pos0 + 4);
            }
            const uint32_t id[G] = {ua.x, ua.y, ua.z, ua.w, uc.x, uc.y, uc.z, uc.w};
            Row A[G], Bv[G];
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const bool bad = id[k] >= (uint32_t)DefaultLevels::codebook;
                nbad += bad ? 1 : 0;
                const uint32_t lo = id[k] & 511u, hi = bad ? 0u : (id[k] >> 9);
                const uint32_t h5 = (hi * 52429u) >> 18, h25 = (hi * 5243u) >> 17;
                const float na = bad ? qnan : 0.0f;
                A[k] = CodeRow<T>::make(((int)(lo & 7) - 4) * 0.25f + na, ((int)((lo >> 3) & 7) - 4) * 0.25f + na,
                                        ((int)(lo >> 6) - 4) * 0.25f + na);
                Bv[k] = CodeRow<T>::make(((int)(hi - 5 * h5) - 2) * 0.5f + na, ((int)(h5 - 5 * h25) - 2) * 0.5f + na,
                                         ((int)h25 - 2) * 0.5f + na);
            }
            // the lane's codes as NCH 16-byte chunks in NTHWC order, or 6 planes of 8 (NCTHW)
            if constexpr (sizeof(T) == 2) {
                // bf16: combine 16-bit fields with byte permutes
                auto lo2 = [](uint32_t a, uint32_t c) { return __builtin_amdgcn_perm(c, a, 0x05040100u); };
                auto hi2 = [](uint32_t a, uint32_t c) { return __builtin_amdgcn_perm(c, a, 0x07060302u); };
                if (LAYOUT == CVT_NCTHW) {
                    const long long b = pos0 / npb, rr = pos0 - b * npb;
                    uint4 o[6];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int q0 = 2 * j, q1 = 2 * j + 1;
                        (&o[0].x)[j] = lo2(A[q0].x, A[q1].x);
                        (&o[1].x)[j] = hi2(A[q0].x, A[q1].x);
                        (&o[2].x)[j] = lo2(A[q0].y, A[q1].y);
                        (&o[3].x)[j] = lo2(Bv[q0].x, Bv[q1].x);
                        (&o[4].x)[j] = hi2(Bv[q0].x, Bv[q1].x);
                        (&o[5].x)[j] = lo2(Bv[q0].y, Bv[q1].y);
                    }
#pragma unroll
                    for (int i = 0; i < 6; ++i)
                        st_stream16(codes + ((size_t)b * 6 + i) * npb + rr, o[i]);
                } else {
                    // per position: (c0 c1) (c2 c3) (c4 c5)
                    uint32_t wd[3 * G];
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        wd[3 * k] = A[k].x;
                        wd[3 * k + 1] = lo2(A[k].y, Bv[k].x);
                        wd[3 * k + 2] = __builtin_amdgcn_perm(Bv[k].y, Bv[k].x, 0x05040302u);
                    }
                    if (full) {
#pragma unroll
                        for (int c = 0; c < NCH; ++c)
                            st[lane * NCH + c] = make_uint4(wd[4 * c], wd[4 * c + 1], wd[4 * c + 2], wd[4 * c + 3]);
                        wave_lds_sync();
                        uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)(wave_id * WAVE_POS) * D);
#pragma unroll
                        for (int c = 0; c < NCH; ++c) st_stream16(dst + c * 64 + lane, st[c * 64 + lane]);
                    } else {
                        uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)pos0 * D);
#pragma unroll
                        for (int c = 0; c < NCH; ++c)
                            dst[c] = make_uint4(wd[4 * c], wd[4 * c + 1], wd[4 * c + 2], wd[4 * c + 3]);
                    }
                }
            } else {
                float cv[D][G];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    cv[0][k] = A[k].x; cv[1][k] = A[k].y; cv[2][k] = A[k].z;
                    cv[3][k] = Bv[k].x; cv[4][k] = Bv[k].y; cv[5][k] = Bv[k].z;
                }
                if (LAYOUT == CVT_NCTHW) {
                    const long long b = pos0 / npb, rr = pos0 - b * npb;
#pragma unroll
                    for (int i = 0; i < D; ++i) store8(codes + ((size_t)b * D + i) * npb + rr, cv[i]);
                } else {
                    float flat[D * G];
#pragma unroll
                    for (int k = 0; k < G; ++k)
#pragma unroll
                        for (int i = 0; i < D; ++i) flat[k * D + i] = cv[i][k];
                    if (full) {
#pragma unroll
                        for (int c = 0; c < NCH; ++c) st[lane * NCH + c] = pack16(flat + c * EPC, T());
                        wave_lds_sync();
                        uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)(wave_id * WAVE_POS) * D);
#pragma unroll
                        for (int c = 0; c < NCH; ++c) st_stream16(dst + c * 64 + lane, st[c * 64 + lane]);
                    } else {
                        uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)pos0 * D);
#pragma unroll
                        for (int c = 0; c < NCH; ++c) dst[c] = pack16(flat + c * EPC, T());
                    }
                }
            }
        } else {
            for (long long pos = pos0; pos < total; ++pos) {  // last partial group (< 8 positions)
                const uint32_t v = (uint32_t)idx[pos];
                const bool bad = v >= (uint32_t)DefaultLevels::codebook;
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
        wave_lds_sync();  // this tile's staged reads before the next tile's writes
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
    if (is_default(p) && vec && (LAYOUT == CVT_NTHWC || B <= 65535)) {
        // one 512-position tile per wave; planar latents get one grid row per clip
        const long long span = LAYOUT == CVT_NCTHW ? npb : total;
        const long long nblk = (span + 4 * WAVE_POS - 1) / (4 * WAVE_POS);
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)nblk, LAYOUT == CVT_NCTHW ? (unsigned)B : 1u);
        if (codes)
            hipLaunchKernelGGL((fsq_quantize_default_kernel<T, LAYOUT, true>), grid, dim3(256), 0, s, (const T*)z, idx,
                               (T*)codes, p, npb, total);
        else
            hipLaunchKernelGGL((fsq_quantize_default_kernel<T, LAYOUT, false>), grid, dim3(256), 0, s, (const T*)z, idx,
                               (T*)nullptr, p, npb, total);
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
        hipLaunchKernelGGL((fsq_dequantize_default_kernel<T, LAYOUT>),
                           dim3((unsigned)((total + 4 * WAVE_POS - 1) / (4 * WAVE_POS))),
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
