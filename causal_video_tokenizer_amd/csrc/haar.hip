// 2-level Haar wavelet patcher with the causal first frame, and its inverse.
//
// The transform is the one described in "NVIDIA Cosmos Tokenizer 完全指南",
// section 7.1 (Haar wavelet patching: each DWT level multiplies channels by 8
// and halves T, H and W; the first frame is repeated to keep latent frame 0
// aligned with frame 0; patch size 4 = two levels) and in the
// Cosmos-Tokenize1-CV8x8x8-720p model card, "Model Architecture" (2-level Haar
// at the encoder input, its inverse at the decoder output).
//
// Two orthonormal levels along one axis of a 4-sample block are a 4x4 matrix
// whose rows are 1/2 (1,1,1,1), (1,1,-1,-1), (1,-1,1,-1), (1,-1,-1,1), row
// 2*b1 + b2 holding level-1 band b1 refined by level-2 band b2.  The 3D
// transform of a 4x4x4 block is the Kronecker product of three of them, so
// this kernel evaluates it as unnormalised +-1 butterflies along w, h and t,
// then scales by 1/8 (1/4 in 2D) once; every scale is a power of two and
// exact.  The matrix is symmetric and orthogonal, so the inverse runs the
// same butterflies.
//
// The causal extension is index arithmetic: padded frame p reads input frame
// max(p - 3, 0), so the extended sequence is never materialised.
//
// Mapping: one wavefront per (b, t', h', run of 64 w' positions); lane = w'.
// Each lane loads the 4 x 4 x 4 block of every input channel with 8-byte
// (bf16) or 16-byte (fp32) row loads, so each load instruction covers 512 or
// 1024 contiguous bytes of a pixel row.  For the NTHWC coefficient layout the
// 64 x (64C) output tile is transposed through LDS (rows padded by one dword so
// the per-lane scattered writes hit distinct banks) and written as contiguous
// dwords; the inverse stages its NTHWC input the same way.
#include "cvt_internal.h"

namespace cvt {
namespace {

__device__ __forceinline__ void packet4(float& a, float& b, float& c, float& d) {
    const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
    a = s0 + s1;
    b = s0 - s1;
    c = d0 + d1;
    d = d0 - d1;
}

__device__ __forceinline__ void load4(const uint16_t* p, float* v) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_lo(u.x);
    v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y);
    v[3] = bf16_hi(u.y);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x;
    v[1] = u.y;
    v[2] = u.z;
    v[3] = u.w;
}
__device__ __forceinline__ void store4(uint16_t* p, const float* v) {
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

// Output channel of packet rows (rt, rh, rw) for input channel c.
template <int NF>
__device__ __forceinline__ int coef_channel(int rt, int rh, int rw, int c, int C) {
    if (NF == 4) {
        const int s1 = ((rt >> 1) << 2) | ((rh >> 1) << 1) | (rw >> 1);
        const int s2 = ((rt & 1) << 2) | ((rh & 1) << 1) | (rw & 1);
        return s2 * 8 * C + s1 * C + c;
    } else {
        const int s1 = ((rh >> 1) << 1) | (rw >> 1);
        const int s2 = ((rh & 1) << 1) | (rw & 1);
        return s2 * 4 * C + s1 * C + c;
    }
}

struct WaveTile {
    int b, tq, hq, chunk, wq;
    bool valid;
};

__device__ __forceinline__ WaveTile decode_tile(int Tq, int Hq, int Wq, int nchunk) {
    WaveTile w;
    long long item = blockIdx.x;
    w.chunk = (int)(item % nchunk);
    item /= nchunk;
    w.hq = (int)(item % Hq);
    item /= Hq;
    w.tq = (int)(item % Tq);
    w.b = (int)(item / Tq);
    w.wq = w.chunk * 64 + (int)threadIdx.x;
    w.valid = w.wq < Wq;
    return w;
}

// NF = 4: 3D (two levels along t, h, w); NF = 1: 2D per frame.
// CT > 0: compile-time channel count; CT = 0: runtime C.
template <typename Tin, typename Tout, int NF, int LAYOUT, int CT>
__global__ __launch_bounds__(64) void haar_fwd_kernel(const Tin* __restrict__ x, Tout* __restrict__ y,
                                                      int C_rt, int T, int H, int W, int Tq, int Hq,
                                                      int Wq, int nchunk, int stage) {
    extern __shared__ uint32_t lds[];
    const int C = CT > 0 ? CT : C_rt;
    const WaveTile tile = decode_tile(Tq, Hq, Wq, nchunk);
    const int lane = threadIdx.x;
    const int wq_ld = tile.valid ? tile.wq : (Wq - 1);  // keep loads in bounds
    const int NCH = (NF == 4 ? 64 : 16) * C;
    const float scale = NF == 4 ? 0.125f : 0.25f;
    const int rowwords = NCH * (int)sizeof(Tout) / 4;
    const int stride = rowwords + 1;
    uint8_t* lds_row = reinterpret_cast<uint8_t*>(lds) + (size_t)lane * stride * 4;

    constexpr int kUnrollC = CT > 0 ? CT : 1;
#pragma unroll kUnrollC
    for (int cr = 0; cr < C; ++cr) {
        {
            float v[NF][4][4];
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int src = NF == 4 ? max(4 * tile.tq + f - 3, 0) : tile.tq;
                const Tin* base = x + (((size_t)(tile.b * C + cr) * T + src) * H + 4 * tile.hq) * W + 4 * wq_ld;
#pragma unroll
                for (int r = 0; r < 4; ++r) load4(base + (size_t)r * W, v[f][r]);
            }
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int r = 0; r < 4; ++r) packet4(v[f][r][0], v[f][r][1], v[f][r][2], v[f][r][3]);
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int k = 0; k < 4; ++k) packet4(v[f][0][k], v[f][1][k], v[f][2][k], v[f][3][k]);
            if constexpr (NF == 4) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int k = 0; k < 4; ++k) packet4(v[0][r][k], v[1][r][k], v[2][r][k], v[3][r][k]);
            }
#pragma unroll
            for (int rt = 0; rt < NF; ++rt)
#pragma unroll
                for (int rh = 0; rh < 4; ++rh)
#pragma unroll
                    for (int rw = 0; rw < 4; ++rw) {
                        const int ch = coef_channel<NF>(rt, rh, rw, cr, C);
                        const float val = v[rt][rh][rw] * scale;
                        if (LAYOUT == CVT_NCTHW) {
                            if (tile.valid)
                                store1(y + ((((size_t)tile.b * NCH + ch) * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq, val);
                        } else if (stage) {
                            store1(reinterpret_cast<Tout*>(lds_row) + ch, val);
                        } else if (tile.valid) {
                            store1(y + ((((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq) * NCH + ch, val);
                        }
                    }
        }
    }

    if (LAYOUT == CVT_NTHWC && stage) {
        __syncthreads();
        const int nvalid = min(64, Wq - tile.chunk * 64);
        const int total = nvalid * rowwords;
        uint32_t* dst = reinterpret_cast<uint32_t*>(
            y + ((((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq + (size_t)tile.chunk * 64) * NCH);
        int row = lane / rowwords, col = lane - (lane / rowwords) * rowwords;
        for (int w = lane; w < total; w += 64) {
            dst[w] = lds[row * stride + col];
            col += 64;
            while (col >= rowwords) {
                col -= rowwords;
                ++row;
            }
        }
    }
}

template <typename Tin, typename Tout, int NF, int LAYOUT, int CT>
__global__ __launch_bounds__(64) void haar_inv_kernel(const Tin* __restrict__ y, Tout* __restrict__ x,
                                                      int C_rt, int T, int H, int W, int Tq, int Hq,
                                                      int Wq, int nchunk, int stage) {
    extern __shared__ uint32_t lds[];
    const int C = CT > 0 ? CT : C_rt;
    const WaveTile tile = decode_tile(Tq, Hq, Wq, nchunk);
    const int lane = threadIdx.x;
    const int NCH = (NF == 4 ? 64 : 16) * C;
    const float scale = NF == 4 ? 0.125f : 0.25f;
    const int rowwords = NCH * (int)sizeof(Tin) / 4;
    const int stride = rowwords + 1;
    const size_t pos = (((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq;

    if (LAYOUT == CVT_NTHWC && stage) {
        const int nvalid = min(64, Wq - tile.chunk * 64);
        const int total = nvalid * rowwords;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(y + (pos + (size_t)tile.chunk * 64) * NCH);
        int row = lane / rowwords, col = lane - (lane / rowwords) * rowwords;
        for (int w = lane; w < total; w += 64) {
            lds[row * stride + col] = src[w];
            col += 64;
            while (col >= rowwords) {
                col -= rowwords;
                ++row;
            }
        }
        __syncthreads();
    }
    if (!tile.valid) return;
    const Tin* lds_row = reinterpret_cast<const Tin*>(reinterpret_cast<const uint8_t*>(lds) + (size_t)lane * stride * 4);

    constexpr int kUnrollC = CT > 0 ? CT : 1;
#pragma unroll kUnrollC
    for (int cr = 0; cr < C; ++cr) {
        {
            float v[NF][4][4];
#pragma unroll
            for (int rt = 0; rt < NF; ++rt)
#pragma unroll
                for (int rh = 0; rh < 4; ++rh)
#pragma unroll
                    for (int rw = 0; rw < 4; ++rw) {
                        const int ch = coef_channel<NF>(rt, rh, rw, cr, C);
                        float val;
                        if (LAYOUT == CVT_NCTHW)
                            val = load1(y + ((((size_t)tile.b * NCH + ch) * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq);
                        else if (stage)
                            val = load1(lds_row + ch);
                        else
                            val = load1(y + (pos + tile.wq) * NCH + ch);
                        v[rt][rh][rw] = val;
                    }
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int r = 0; r < 4; ++r) packet4(v[f][r][0], v[f][r][1], v[f][r][2], v[f][r][3]);
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int k = 0; k < 4; ++k) packet4(v[f][0][k], v[f][1][k], v[f][2][k], v[f][3][k]);
            if constexpr (NF == 4) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int k = 0; k < 4; ++k) packet4(v[0][r][k], v[1][r][k], v[2][r][k], v[3][r][k]);
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int t = NF == 4 ? 4 * tile.tq + f - 3 : tile.tq;  // drop the 3 leading padded frames
                if (t < 0) continue;
                Tout* base = x + (((size_t)(tile.b * C + cr) * T + t) * H + 4 * tile.hq) * W + 4 * tile.wq;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = v[f][r][k] * scale;
                    store4(base + (size_t)r * W, o);
                }
            }
        }
    }
}

constexpr int kLdsLimit = 64 * 1024;

template <typename Tin, typename Tout, int NF, int LAYOUT>
hipError_t launch_fwd_t(const void* x, void* y, int B, int C, int T, int H, int W, hipStream_t s) {
    const int Tq = NF == 4 ? 1 + (T - 1) / 4 : T, Hq = H / 4, Wq = W / 4;
    const int nchunk = (Wq + 63) / 64;
    const long long nblk = (long long)B * Tq * Hq * nchunk;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int NCH = (NF == 4 ? 64 : 16) * C;
    const size_t lds_bytes = (size_t)64 * (NCH * sizeof(Tout) / 4 + 1) * 4;
    const int stage = (LAYOUT == CVT_NTHWC) && lds_bytes <= (size_t)kLdsLimit;
    const size_t shmem = stage ? lds_bytes : 0;
    if (C == 3)
        hipLaunchKernelGGL((haar_fwd_kernel<Tin, Tout, NF, LAYOUT, 3>), dim3((unsigned)nblk), dim3(64), shmem, s,
                           (const Tin*)x, (Tout*)y, C, T, H, W, Tq, Hq, Wq, nchunk, stage);
    else
        hipLaunchKernelGGL((haar_fwd_kernel<Tin, Tout, NF, LAYOUT, 0>), dim3((unsigned)nblk), dim3(64), shmem, s,
                           (const Tin*)x, (Tout*)y, C, T, H, W, Tq, Hq, Wq, nchunk, stage);
    return hipGetLastError();
}

template <typename Tin, typename Tout, int NF, int LAYOUT>
hipError_t launch_inv_t(const void* y, void* x, int B, int C, int T, int H, int W, hipStream_t s) {
    const int Tq = NF == 4 ? (T + 3) / 4 : T, Hq = H / 4, Wq = W / 4;
    const int nchunk = (Wq + 63) / 64;
    const long long nblk = (long long)B * Tq * Hq * nchunk;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int NCH = (NF == 4 ? 64 : 16) * C;
    const size_t lds_bytes = (size_t)64 * (NCH * sizeof(Tin) / 4 + 1) * 4;
    const int stage = (LAYOUT == CVT_NTHWC) && lds_bytes <= (size_t)kLdsLimit;
    const size_t shmem = stage ? lds_bytes : 0;
    if (C == 3)
        hipLaunchKernelGGL((haar_inv_kernel<Tin, Tout, NF, LAYOUT, 3>), dim3((unsigned)nblk), dim3(64), shmem, s,
                           (const Tin*)y, (Tout*)x, C, T, H, W, Tq, Hq, Wq, nchunk, stage);
    else
        hipLaunchKernelGGL((haar_inv_kernel<Tin, Tout, NF, LAYOUT, 0>), dim3((unsigned)nblk), dim3(64), shmem, s,
                           (const Tin*)y, (Tout*)x, C, T, H, W, Tq, Hq, Wq, nchunk, stage);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t fwd_by_shape(const void* x, void* y, int layout, int B, int C, int T, int H, int W, int tl, hipStream_t s) {
    if (tl == 2)
        return layout == CVT_NTHWC ? launch_fwd_t<Tin, Tout, 4, CVT_NTHWC>(x, y, B, C, T, H, W, s)
                                   : launch_fwd_t<Tin, Tout, 4, CVT_NCTHW>(x, y, B, C, T, H, W, s);
    return layout == CVT_NTHWC ? launch_fwd_t<Tin, Tout, 1, CVT_NTHWC>(x, y, B, C, T, H, W, s)
                               : launch_fwd_t<Tin, Tout, 1, CVT_NCTHW>(x, y, B, C, T, H, W, s);
}

template <typename Tin, typename Tout>
hipError_t inv_by_shape(const void* y, void* x, int layout, int B, int C, int T, int H, int W, int tl, hipStream_t s) {
    if (tl == 2)
        return layout == CVT_NTHWC ? launch_inv_t<Tin, Tout, 4, CVT_NTHWC>(y, x, B, C, T, H, W, s)
                                   : launch_inv_t<Tin, Tout, 4, CVT_NCTHW>(y, x, B, C, T, H, W, s);
    return layout == CVT_NTHWC ? launch_inv_t<Tin, Tout, 1, CVT_NTHWC>(y, x, B, C, T, H, W, s)
                               : launch_inv_t<Tin, Tout, 1, CVT_NCTHW>(y, x, B, C, T, H, W, s);
}

}  // namespace

hipError_t launch_haar_fwd(const void* x, int x_dtype, void* y, int y_dtype, int y_layout, int B, int C,
                           int T, int H, int W, int temporal_levels, hipStream_t s) {
    if (x_dtype == CVT_BF16) {
        return y_dtype == CVT_BF16 ? fwd_by_shape<uint16_t, uint16_t>(x, y, y_layout, B, C, T, H, W, temporal_levels, s)
                                   : fwd_by_shape<uint16_t, float>(x, y, y_layout, B, C, T, H, W, temporal_levels, s);
    }
    return y_dtype == CVT_BF16 ? fwd_by_shape<float, uint16_t>(x, y, y_layout, B, C, T, H, W, temporal_levels, s)
                               : fwd_by_shape<float, float>(x, y, y_layout, B, C, T, H, W, temporal_levels, s);
}

hipError_t launch_haar_inv(const void* y, int y_dtype, int y_layout, void* x, int x_dtype, int B, int C,
                           int T, int H, int W, int temporal_levels, hipStream_t s) {
    if (y_dtype == CVT_BF16) {
        return x_dtype == CVT_BF16 ? inv_by_shape<uint16_t, uint16_t>(y, x, y_layout, B, C, T, H, W, temporal_levels, s)
                                   : inv_by_shape<uint16_t, float>(y, x, y_layout, B, C, T, H, W, temporal_levels, s);
    }
    return x_dtype == CVT_BF16 ? inv_by_shape<float, uint16_t>(y, x, y_layout, B, C, T, H, W, temporal_levels, s)
                               : inv_by_shape<float, float>(y, x, y_layout, B, C, T, H, W, temporal_levels, s);
}

}  // namespace cvt
