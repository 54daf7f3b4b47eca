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
// max(p - pad, 0) with pad = 3, so the extended sequence is never materialised.
// A continuation chunk of a stream (pad = 0) has no leading copies: its latent
// frame j is frames 4j .. 4j+3, exactly the latent frame the whole clip gives there.
//
// Sliding windows (WM != 0): the kernels can also read one window of a longer clip as the
// padded window the tokenizer accepts (time mirrored about the window's last frame, zero
// rows and columns past the frame) and write the inverse straight back into the clip,
// cropped, so neither the padded window nor its reconstruction is materialised.  WM = 1
// when the clip's width is a multiple of 4 (a 4-pixel group is wholly inside the clip's
// row or wholly past it), WM = 2 for rows of any length, accessed element by element.
//
// Mapping: one wavefront per (b, t', h', run of 64 w' positions); lane = w'.
// Each lane loads the 4 x 4 x 4 block of every input channel with 8-byte
// (bf16) or 16-byte (fp32) streaming row loads, so each load instruction covers
// 512 or 1024 contiguous bytes of a pixel row.  For the NTHWC coefficient layout
// with C = 3 the 64 x (64C) output tile goes through LDS (rows padded by 16 bytes so
// the 128-bit row accesses of 16 lanes hit distinct banks) and leaves as contiguous
// 16-byte stores; the inverse stages its NTHWC input the same way.  Other channel
// counts and layouts use the generic kernels at the end of the file.
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

// Window access: 4 pixels of row h from column w of a clip frame plane; rows >= H and
// columns >= W of the padded window read as zero and are not written.
template <int WM, typename T>
__device__ __forceinline__ void load4_win(const T* plane, int h, int w, const ClipWindow& win, float* v) {
    v[0] = v[1] = v[2] = v[3] = 0.0f;
    if (h >= win.H || w >= win.W) return;
    const T* p = plane + (size_t)h * win.W + w;
    if (WM == 1) {
        load4(p, v);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (w + k < win.W) v[k] = load1(p + k);
    }
}
template <int WM, typename T>
__device__ __forceinline__ void store4_win(T* plane, int h, int w, const ClipWindow& win, const float* v) {
    if (h >= win.H || w >= win.W) return;
    T* p = plane + (size_t)h * win.W + w;
    if (WM == 1) {
        store4(p, v);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (w + k < win.W) store1(p + k, v[k]);
    }
}
// Clip frame plane of padded (forward) or cropped (inverse) window frame p, channel plane bc.
template <typename T>
__device__ __forceinline__ T* clip_plane(T* x, int bc, int frame, const ClipWindow& win) {
    return x + ((size_t)bc * win.T + win.t0 + frame) * win.H * (size_t)win.W;
}

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

// Element traits: bytes per element and 16-byte packing.
template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int per16 = 8;  // elements per 16 bytes
};
template <>
struct Elem<float> {
    static constexpr int per16 = 4;
};

// Pack 4 (bf16: 8) consecutive floats of `v` into one 16-byte word.
__device__ __forceinline__ uint4 pack16(const float* v, uint16_t*) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ uint4 pack16(const float* v, float*) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}
// Unpack one 16-byte word into 8 (bf16) or 4 (fp32) floats.
__device__ __forceinline__ void unpack16(const uint4 u, float* v, const uint16_t*) {
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void unpack16(const uint4 u, float* v, const float*) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y); v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}

// Raw 4-element row segment as loaded from memory.
template <typename T>
struct Row4;
template <>
struct Row4<uint16_t> {
    uint2 u;
    __device__ void load(const uint16_t* p) { u = ld_stream8(p); }
    __device__ void get(float* v) const {
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    }
};
template <>
struct Row4<float> {
    float4 u;
    __device__ void load(const float* p) {
        const uint4 w = ld_stream16(p);
        u = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
    }
    __device__ void get(float* v) const { v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w; }
};

// Forward/inverse transform of one channel's 4 x 4 x 4 (NF = 4) or 4 x 4 (NF = 1) block in place.
template <int NF>
__device__ __forceinline__ void block_transform(float (&v)[NF][4][4]) {
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
}

// ---------------------------------------------------------------------------------------------
// Fast forward kernel: compile-time channel count CT, NTHWC output staged through LDS.
// Each lane keeps all 64*CT coefficients of its position in registers, packs them
// into 16-byte words in channel order and writes its LDS row with 128-bit stores;
// the wave then copies its 64 contiguous rows out with 16-byte coalesced stores.
// LDS row stride = row bytes + 16, so the 128-bit row accesses of 16 lanes fall
// on distinct banks.
template <typename Tin, typename Tout, int NF, int CT, int WM>
__global__ __launch_bounds__(64) void haar_fwd_staged_kernel(const Tin* __restrict__ x, Tout* __restrict__ y,
                                                             int T, int H, int W, int Tq, int Hq, int Wq,
                                                             int nchunk, int pad, ClipWindow win) {
    static_assert(WM == 0 || WM == 1, "rows of any length take the generic kernel");
    constexpr int C = CT;
    constexpr int G = NF == 4 ? 64 : 16;
    constexpr int NCH = G * C;
    constexpr int P16 = Elem<Tout>::per16;
    constexpr int ROW16 = NCH / P16;          // 16-byte words per row
    constexpr int STRIDE = (ROW16 + 1) * 16;  // bytes
    static_assert(NCH % P16 == 0, "row must be a whole number of 16-byte words");
    __shared__ __attribute__((aligned(16))) uint8_t lds[64 * STRIDE];
    const float scale = NF == 4 ? 0.125f : 0.25f;

    const WaveTile tile = decode_tile(Tq, Hq, Wq, nchunk);
    const int lane = threadIdx.x;
    const int wq_ld = tile.valid ? tile.wq : (Wq - 1);

    // 1. all loads of the block, every channel
    Row4<Tin> raw[C][NF][4];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int src = NF == 4 ? max(4 * tile.tq + f - pad, 0) : tile.tq;
            if constexpr (WM == 0) {
                const Tin* base = x + (((size_t)(tile.b * C + c) * T + src) * H + 4 * tile.hq) * W + 4 * wq_ld;
#pragma unroll
                for (int r = 0; r < 4; ++r) raw[c][f][r].load(base + (size_t)r * W);
            } else {
                // rows past the clip's frame and 4-pixel groups past its width load a clamped, valid
                // group and are zeroed where the transform reads them: the loads stay unconditional,
                // so all of them are in flight together
                const Tin* plane = clip_plane(x, tile.b * C + c, mirror_frame(src, win.nt), win);
                const int wl = min(4 * wq_ld, win.W - 4);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    raw[c][f][r].load(plane + (size_t)min(4 * tile.hq + r, win.H - 1) * win.W + wl);
            }
        }

    // 2. transform, in output channel order
    float out[NCH];
    bool okr[4];  // WM: row r of the block lies inside the clip's frame (and the lane's group inside its width)
#pragma unroll
    for (int r = 0; r < 4; ++r) okr[r] = WM == 0 || (4 * tile.hq + r < win.H && 4 * wq_ld < win.W);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        float v[NF][4][4];
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                raw[c][f][r].get(v[f][r]);
                if constexpr (WM != 0) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[f][r][k] = okr[r] ? v[f][r][k] : 0.0f;
                }
            }
        block_transform<NF>(v);
#pragma unroll
        for (int rt = 0; rt < NF; ++rt)
#pragma unroll
            for (int rh = 0; rh < 4; ++rh)
#pragma unroll
                for (int rw = 0; rw < 4; ++rw) out[coef_channel<NF>(rt, rh, rw, c, C)] = v[rt][rh][rw] * scale;
    }

    // 3. row -> LDS (128-bit stores), then coalesced 16-byte copy-out of the wave's rows
    uint8_t* row = lds + lane * STRIDE;
#pragma unroll
    for (int j = 0; j < ROW16; ++j)
        *reinterpret_cast<uint4*>(row + 16 * j) = pack16(out + j * P16, (Tout*)nullptr);
    __syncthreads();
    const int nvalid = min(64, Wq - tile.chunk * 64);
    const int total = nvalid * ROW16;
    uint4* dst = reinterpret_cast<uint4*>(
        y + ((((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq + (size_t)tile.chunk * 64) * NCH);
#pragma unroll
    for (int i = 0; i < ROW16; ++i) {
        const int q = lane + 64 * i;
        if (q < total) {
            const int r = q / ROW16, c16 = q - (q / ROW16) * ROW16;
            dst[q] = *reinterpret_cast<const uint4*>(lds + r * STRIDE + 16 * c16);
        }
    }
}

// Fast inverse kernel: compile-time CT, NTHWC input staged through LDS with
// coalesced 16-byte streaming loads; each lane reads its row back with 128-bit
// LDS reads.
template <typename Tin, typename Tout, int NF, int CT, int WM>
__global__ __launch_bounds__(64) void haar_inv_staged_kernel(const Tin* __restrict__ y, Tout* __restrict__ x,
                                                             int T, int H, int W, int Tq, int Hq, int Wq,
                                                             int nchunk, int pad, ClipWindow win) {
    static_assert(WM == 0 || WM == 1, "rows of any length take the generic kernel");
    constexpr int C = CT;
    constexpr int G = NF == 4 ? 64 : 16;
    constexpr int NCH = G * C;
    constexpr int P16 = Elem<Tin>::per16;
    constexpr int ROW16 = NCH / P16;
    constexpr int STRIDE = (ROW16 + 1) * 16;
    static_assert(NCH % P16 == 0, "row must be a whole number of 16-byte words");
    __shared__ __attribute__((aligned(16))) uint8_t lds[64 * STRIDE];
    const float scale = NF == 4 ? 0.125f : 0.25f;

    const WaveTile tile = decode_tile(Tq, Hq, Wq, nchunk);
    const int lane = threadIdx.x;
    const int nvalid = min(64, Wq - tile.chunk * 64);
    const int total = nvalid * ROW16;
    const uint4* src = reinterpret_cast<const uint4*>(
        y + ((((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq + (size_t)tile.chunk * 64) * NCH);

    // 1. coalesced 16-byte loads of the wave's rows, all in flight, then LDS.  On a
    // partial run the index is clamped: the duplicate words land in LDS rows that
    // belong to positions past the end, which no valid lane reads.
    uint4 stage[ROW16];
#pragma unroll
    for (int i = 0; i < ROW16; ++i) stage[i] = ld_stream16(src + min(lane + 64 * i, total - 1));
#pragma unroll
    for (int i = 0; i < ROW16; ++i) {
        const int q = lane + 64 * i;
        const int r = q / ROW16, c16 = q - (q / ROW16) * ROW16;
        *reinterpret_cast<uint4*>(lds + r * STRIDE + 16 * c16) = stage[i];
    }
    __syncthreads();
    if (!tile.valid) return;

    // 2. this lane's row
    float coef[NCH];
    const uint8_t* row = lds + lane * STRIDE;
#pragma unroll
    for (int j = 0; j < ROW16; ++j) unpack16(*reinterpret_cast<const uint4*>(row + 16 * j), coef + j * P16, (const Tin*)nullptr);

    // 3. per channel: inverse transform and 8/16-byte pixel-row stores
#pragma unroll
    for (int c = 0; c < C; ++c) {
        float v[NF][4][4];
#pragma unroll
        for (int rt = 0; rt < NF; ++rt)
#pragma unroll
            for (int rh = 0; rh < 4; ++rh)
#pragma unroll
                for (int rw = 0; rw < 4; ++rw) v[rt][rh][rw] = coef[coef_channel<NF>(rt, rh, rw, c, C)];
        block_transform<NF>(v);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int t = NF == 4 ? 4 * tile.tq + f - pad : tile.tq;  // drop the leading padded frames
            if (t < 0) continue;
            if constexpr (WM == 0) {
                Tout* base = x + (((size_t)(tile.b * C + c) * T + t) * H + 4 * tile.hq) * W + 4 * tile.wq;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = v[f][r][k] * scale;
                    store4(base + (size_t)r * W, o);
                }
            } else {
                if (t >= win.nt) continue;  // frames of the time padding are cropped
                Tout* plane = clip_plane(x, tile.b * C + c, t, win);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = v[f][r][k] * scale;
                    store4_win<WM>(plane, 4 * tile.hq + r, 4 * tile.wq, win, o);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Generic kernels (runtime channel count, either layout, no staging): correct for
// every shape the ABI accepts; used when the fast kernels do not apply.
template <typename Tin, typename Tout, int NF, int LAYOUT, int WM>
__global__ __launch_bounds__(64) void haar_fwd_generic_kernel(const Tin* __restrict__ x, Tout* __restrict__ y, int C,
                                                              int T, int H, int W, int Tq, int Hq, int Wq,
                                                              int nchunk, int pad, ClipWindow win) {
    const WaveTile tile = decode_tile(Tq, Hq, Wq, nchunk);
    if (!tile.valid) return;
    const int NCH = (NF == 4 ? 64 : 16) * C;
    const float scale = NF == 4 ? 0.125f : 0.25f;
    for (int c = 0; c < C; ++c) {
        float v[NF][4][4];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int src = NF == 4 ? max(4 * tile.tq + f - pad, 0) : tile.tq;
            if constexpr (WM == 0) {
                const Tin* base = x + (((size_t)(tile.b * C + c) * T + src) * H + 4 * tile.hq) * W + 4 * tile.wq;
#pragma unroll
                for (int r = 0; r < 4; ++r) load4(base + (size_t)r * W, v[f][r]);
            } else {
                const Tin* plane = clip_plane(x, tile.b * C + c, mirror_frame(src, win.nt), win);
#pragma unroll
                for (int r = 0; r < 4; ++r) load4_win<WM>(plane, 4 * tile.hq + r, 4 * tile.wq, win, v[f][r]);
            }
        }
        block_transform<NF>(v);
#pragma unroll
        for (int rt = 0; rt < NF; ++rt)
#pragma unroll
            for (int rh = 0; rh < 4; ++rh)
#pragma unroll
                for (int rw = 0; rw < 4; ++rw) {
                    const int ch = coef_channel<NF>(rt, rh, rw, c, C);
                    const size_t off = LAYOUT == CVT_NCTHW
                        ? ((((size_t)tile.b * NCH + ch) * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq
                        : ((((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq) * NCH + ch;
                    store1(y + off, v[rt][rh][rw] * scale);
                }
    }
}

template <typename Tin, typename Tout, int NF, int LAYOUT, int WM>
__global__ __launch_bounds__(64) void haar_inv_generic_kernel(const Tin* __restrict__ y, Tout* __restrict__ x, int C,
                                                              int T, int H, int W, int Tq, int Hq, int Wq,
                                                              int nchunk, int pad, ClipWindow win) {
    const WaveTile tile = decode_tile(Tq, Hq, Wq, nchunk);
    if (!tile.valid) return;
    const int NCH = (NF == 4 ? 64 : 16) * C;
    const float scale = NF == 4 ? 0.125f : 0.25f;
    for (int c = 0; c < C; ++c) {
        float v[NF][4][4];
#pragma unroll
        for (int rt = 0; rt < NF; ++rt)
#pragma unroll
            for (int rh = 0; rh < 4; ++rh)
#pragma unroll
                for (int rw = 0; rw < 4; ++rw) {
                    const int ch = coef_channel<NF>(rt, rh, rw, c, C);
                    const size_t off = LAYOUT == CVT_NCTHW
                        ? ((((size_t)tile.b * NCH + ch) * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq
                        : ((((size_t)tile.b * Tq + tile.tq) * Hq + tile.hq) * Wq + tile.wq) * NCH + ch;
                    v[rt][rh][rw] = load1(y + off);
                }
        block_transform<NF>(v);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int t = NF == 4 ? 4 * tile.tq + f - pad : tile.tq;
            if (t < 0) continue;
            if constexpr (WM == 0) {
                Tout* base = x + (((size_t)(tile.b * C + c) * T + t) * H + 4 * tile.hq) * W + 4 * tile.wq;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = v[f][r][k] * scale;
                    store4(base + (size_t)r * W, o);
                }
            } else {
                if (t >= win.nt) continue;
                Tout* plane = clip_plane(x, tile.b * C + c, t, win);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) o[k] = v[f][r][k] * scale;
                    store4_win<WM>(plane, 4 * tile.hq + r, 4 * tile.wq, win, o);
                }
            }
        }
    }
}

// pad: leading copies of frame 0 (3 for a clip or a stream's first chunk, 0 for a
// continuation chunk of 4k frames).  T, H, W: the (padded window's) pixel sizes.
template <typename Tin, typename Tout, int NF, int LAYOUT, int WM>
hipError_t launch_fwd_t(const void* x, void* y, int B, int C, int T, int H, int W, int pad, const ClipWindow& win,
                        hipStream_t s) {
    const int Tq = NF == 4 ? (T + pad) / 4 : T, Hq = H / 4, Wq = W / 4;
    const int nchunk = (Wq + 63) / 64;
    const long long nblk = (long long)B * Tq * Hq * nchunk;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    bool staged = false;
    if constexpr (LAYOUT == CVT_NTHWC && WM != 2) {
        if (C == 3) {
            hipLaunchKernelGGL((haar_fwd_staged_kernel<Tin, Tout, NF, 3, WM>), dim3((unsigned)nblk), dim3(64), 0, s,
                               (const Tin*)x, (Tout*)y, T, H, W, Tq, Hq, Wq, nchunk, pad, win);
            staged = true;
        }
    }
    if (!staged)
        hipLaunchKernelGGL((haar_fwd_generic_kernel<Tin, Tout, NF, LAYOUT, WM>), dim3((unsigned)nblk), dim3(64), 0, s,
                           (const Tin*)x, (Tout*)y, C, T, H, W, Tq, Hq, Wq, nchunk, pad, win);
    return hipGetLastError();
}

template <typename Tin, typename Tout, int NF, int LAYOUT, int WM>
hipError_t launch_inv_t(const void* y, void* x, int B, int C, int T, int H, int W, int pad, const ClipWindow& win,
                        hipStream_t s) {
    const int Tq = NF == 4 ? (T + pad) / 4 : T, Hq = H / 4, Wq = W / 4;
    const int nchunk = (Wq + 63) / 64;
    const long long nblk = (long long)B * Tq * Hq * nchunk;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    bool staged = false;
    if constexpr (LAYOUT == CVT_NTHWC && WM != 2) {
        if (C == 3) {
            hipLaunchKernelGGL((haar_inv_staged_kernel<Tin, Tout, NF, 3, WM>), dim3((unsigned)nblk), dim3(64), 0, s,
                               (const Tin*)y, (Tout*)x, T, H, W, Tq, Hq, Wq, nchunk, pad, win);
            staged = true;
        }
    }
    if (!staged)
        hipLaunchKernelGGL((haar_inv_generic_kernel<Tin, Tout, NF, LAYOUT, WM>), dim3((unsigned)nblk), dim3(64), 0, s,
                           (const Tin*)y, (Tout*)x, C, T, H, W, Tq, Hq, Wq, nchunk, pad, win);
    return hipGetLastError();
}

// Window mode: 0 = the whole input, 1 = a window of a clip whose width is a multiple of 4,
// 2 = a window of a clip with rows of any length.
int window_mode(const ClipWindow* win) { return !win ? 0 : (win->W % 4 == 0 ? 1 : 2); }

// tl: 0 = per-frame 2D patcher; 2 = 3D with the causal first frame; 3 = 3D continuation
// chunk (frames 4j .. 4j+3 form latent frame j, no leading copies)
template <bool FWD, typename Tin, typename Tout, int NF, int LAYOUT, int WM>
hipError_t launch_dir(const void* a, void* b, int B, int C, int T, int H, int W, int pad, const ClipWindow& w,
                      hipStream_t s) {
    if constexpr (FWD) return launch_fwd_t<Tin, Tout, NF, LAYOUT, WM>(a, b, B, C, T, H, W, pad, w, s);
    else return launch_inv_t<Tin, Tout, NF, LAYOUT, WM>(a, b, B, C, T, H, W, pad, w, s);
}

template <bool FWD, typename Tin, typename Tout, int NF, int LAYOUT>
hipError_t dispatch_wm(const void* a, void* b, int B, int C, int T, int H, int W, int pad, const ClipWindow* win,
                       hipStream_t s) {
    const ClipWindow w = win ? *win : ClipWindow{T, H, W, 0, T};
    switch (window_mode(win)) {
        case 0: return launch_dir<FWD, Tin, Tout, NF, LAYOUT, 0>(a, b, B, C, T, H, W, pad, w, s);
        case 1: return launch_dir<FWD, Tin, Tout, NF, LAYOUT, 1>(a, b, B, C, T, H, W, pad, w, s);
        default: return launch_dir<FWD, Tin, Tout, NF, LAYOUT, 2>(a, b, B, C, T, H, W, pad, w, s);
    }
}

template <bool FWD, typename Tin, typename Tout>
hipError_t by_shape(const void* a, void* b, int layout, int B, int C, int T, int H, int W, int tl, const ClipWindow* win,
                    hipStream_t s) {
    if (tl == 2 || tl == 3) {
        const int pad = tl == 2 ? 3 : 0;
        return layout == CVT_NTHWC ? dispatch_wm<FWD, Tin, Tout, 4, CVT_NTHWC>(a, b, B, C, T, H, W, pad, win, s)
                                   : dispatch_wm<FWD, Tin, Tout, 4, CVT_NCTHW>(a, b, B, C, T, H, W, pad, win, s);
    }
    return layout == CVT_NTHWC ? dispatch_wm<FWD, Tin, Tout, 1, CVT_NTHWC>(a, b, B, C, T, H, W, 0, win, s)
                               : dispatch_wm<FWD, Tin, Tout, 1, CVT_NCTHW>(a, b, B, C, T, H, W, 0, win, s);
}

}  // namespace

hipError_t launch_haar_fwd(const void* x, int x_dtype, void* y, int y_dtype, int y_layout, int B, int C,
                           int T, int H, int W, int temporal_levels, hipStream_t s, const ClipWindow* win) {
    if (x_dtype == CVT_BF16) {
        return y_dtype == CVT_BF16
                   ? by_shape<true, uint16_t, uint16_t>(x, y, y_layout, B, C, T, H, W, temporal_levels, win, s)
                   : by_shape<true, uint16_t, float>(x, y, y_layout, B, C, T, H, W, temporal_levels, win, s);
    }
    return y_dtype == CVT_BF16 ? by_shape<true, float, uint16_t>(x, y, y_layout, B, C, T, H, W, temporal_levels, win, s)
                               : by_shape<true, float, float>(x, y, y_layout, B, C, T, H, W, temporal_levels, win, s);
}

hipError_t launch_haar_inv(const void* y, int y_dtype, int y_layout, void* x, int x_dtype, int B, int C,
                           int T, int H, int W, int temporal_levels, hipStream_t s, const ClipWindow* win) {
    if (y_dtype == CVT_BF16) {
        return x_dtype == CVT_BF16
                   ? by_shape<false, uint16_t, uint16_t>(y, x, y_layout, B, C, T, H, W, temporal_levels, win, s)
                   : by_shape<false, uint16_t, float>(y, x, y_layout, B, C, T, H, W, temporal_levels, win, s);
    }
    return x_dtype == CVT_BF16 ? by_shape<false, float, uint16_t>(y, x, y_layout, B, C, T, H, W, temporal_levels, win, s)
                               : by_shape<false, float, float>(y, x, y_layout, B, C, T, H, W, temporal_levels, win, s);
}

}  // namespace cvt
