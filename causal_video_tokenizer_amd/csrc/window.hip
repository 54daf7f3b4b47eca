// Sliding-window processing of videos of any length and size: pad one window of a clip up
// to the sizes the tokenizer accepts, and crop a processed window back into the clip.
//
// Cosmos Tokenizer guide, section 6.3 (videos of any length): the clip is worked through
// in windows of temporal_window frames; each window is padded with zeros in space and by
// reflection at its last frame in time, reconstructed, cropped back and concatenated.
// Sections 6.1 and 7.3 fix the aligned length of a causal clip: 1 + k*f frames.
//
// Both kernels are pure copies (bit-exact), bound by HBM.  A thread moves one vector of
// V elements (16 bytes where the row length allows, else 8 bytes or single elements);
// blockIdx.x covers one frame plane, blockIdx.y strides over the B*C*frames planes.
#include "cvt_internal.h"

namespace cvt {

namespace {

template <typename E, int V>
struct alignas(sizeof(E) * V) Vec {
    E e[V];
};

struct WinGeom {
    int T, H, W;        // the clip
    int t0, nt;         // the window: frames t0 .. t0 + nt - 1
    int Tp, Hp, Wp;     // the padded window
    int planes;         // frame planes the launch covers (B*C*Tp for pad, B*C*nt for crop)
};

// ALIGNED: W % V == 0, so a vector of the padded row is a vector of the source row (or
// wholly past it).
template <typename E, int V, bool ALIGNED>
__global__ __launch_bounds__(256) void video_pad_kernel(const E* __restrict__ x, E* __restrict__ y, WinGeom g) {
    const int vpr = g.Wp / V;
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (i >= g.Hp * vpr) return;
    const int h = i / vpr, w0 = (i - h * vpr) * V;
    for (int p = blockIdx.y; p < g.planes; p += gridDim.y) {
        const int bc = p / g.Tp, t = p - bc * g.Tp;
        Vec<E, V> v;
#pragma unroll
        for (int e = 0; e < V; ++e) v.e[e] = 0;
        if (h < g.H) {
            const int ts = g.t0 + mirror_frame(t, g.nt);
            const E* src = x + (((size_t)bc * g.T + ts) * g.H + h) * (size_t)g.W;
            if (ALIGNED) {
                if (w0 < g.W) v = *reinterpret_cast<const Vec<E, V>*>(src + w0);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    if (w0 + e < g.W) v.e[e] = src[w0 + e];
            }
        }
        *reinterpret_cast<Vec<E, V>*>(y + ((size_t)p * g.Hp + h) * (size_t)g.Wp + w0) = v;
    }
}

// ALIGNED: W % V == 0 (and Wp % V == 0), so a destination vector is a vector of the padded
// row.  Otherwise a thread moves V consecutive elements of the destination plane, each
// fetched on its own.
template <typename E, int V, bool ALIGNED>
__global__ __launch_bounds__(256) void video_unpad_kernel(const E* __restrict__ y, E* __restrict__ x, WinGeom g) {
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    const int n = g.H * g.W;  // destination plane
    if (i * V >= n) return;
    for (int p = blockIdx.y; p < g.planes; p += gridDim.y) {
        const int bc = p / g.nt, t = p - bc * g.nt;
        const E* src = y + ((size_t)bc * g.Tp + t) * (size_t)g.Hp * g.Wp;
        E* dst = x + ((size_t)bc * g.T + g.t0 + t) * (size_t)n;
        if (ALIGNED) {
            const int vpr = g.W / V;
            const int h = i / vpr, w0 = (i - h * vpr) * V;
            *reinterpret_cast<Vec<E, V>*>(dst + (size_t)h * g.W + w0) =
                *reinterpret_cast<const Vec<E, V>*>(src + (size_t)h * g.Wp + w0);
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int f = i * V + e;
                if (f < n) {
                    const int h = f / g.W, w = f - h * g.W;
                    dst[f] = src[(size_t)h * g.Wp + w];
                }
            }
        }
    }
}

constexpr int WIN_MAX_GRID_Y = 65535;

template <typename E>
hipError_t launch_pad_t(const void* x, void* y, int planes, const WinGeom& g, hipStream_t s) {
    constexpr int V16 = 16 / (int)sizeof(E), V8 = 8 / (int)sizeof(E);
    const E* xs = static_cast<const E*>(x);
    E* ys = static_cast<E*>(y);
    const dim3 block(256);
    const unsigned gy = (unsigned)std::min(planes, WIN_MAX_GRID_Y);
    auto grid = [&](int V) { return dim3((unsigned)(((long long)g.Hp * (g.Wp / V) + 255) / 256), gy); };
    if (g.Wp % V16 == 0) {
        if (g.W % V16 == 0)
            hipLaunchKernelGGL((video_pad_kernel<E, V16, true>), grid(V16), block, 0, s, xs, ys, g);
        else
            hipLaunchKernelGGL((video_pad_kernel<E, V16, false>), grid(V16), block, 0, s, xs, ys, g);
    } else if (g.Wp % V8 == 0) {
        if (g.W % V8 == 0)
            hipLaunchKernelGGL((video_pad_kernel<E, V8, true>), grid(V8), block, 0, s, xs, ys, g);
        else
            hipLaunchKernelGGL((video_pad_kernel<E, V8, false>), grid(V8), block, 0, s, xs, ys, g);
    } else {
        hipLaunchKernelGGL((video_pad_kernel<E, 1, true>), grid(1), block, 0, s, xs, ys, g);
    }
    return hipGetLastError();
}

template <typename E>
hipError_t launch_unpad_t(const void* y, void* x, int planes, const WinGeom& g, hipStream_t s) {
    constexpr int V16 = 16 / (int)sizeof(E), V8 = 8 / (int)sizeof(E);
    const E* ys = static_cast<const E*>(y);
    E* xs = static_cast<E*>(x);
    const dim3 block(256);
    const unsigned gy = (unsigned)std::min(planes, WIN_MAX_GRID_Y);
    auto grid = [&](int V) { return dim3((unsigned)(((long long)g.H * g.W / V + 255) / 256), gy); };
    if (g.W % V16 == 0 && g.Wp % V16 == 0)
        hipLaunchKernelGGL((video_unpad_kernel<E, V16, true>), grid(V16), block, 0, s, ys, xs, g);
    else if (g.W % V8 == 0 && g.Wp % V8 == 0)
        hipLaunchKernelGGL((video_unpad_kernel<E, V8, true>), grid(V8), block, 0, s, ys, xs, g);
    else  // ragged rows: V8 consecutive elements of the destination plane per thread
        hipLaunchKernelGGL((video_unpad_kernel<E, V8, false>),
                           dim3((unsigned)(((long long)g.H * g.W + V8 * 256 - 1) / (V8 * 256)), gy), block, 0, s, ys,
                           xs, g);
    return hipGetLastError();
}

WinGeom win_geom(int T, int H, int W, int t0, int nt, int Tp, int Hp, int Wp, int planes) {
    WinGeom g{};
    g.T = T; g.H = H; g.W = W; g.t0 = t0; g.nt = nt; g.Tp = Tp; g.Hp = Hp; g.Wp = Wp; g.planes = planes;
    return g;
}

}  // namespace

hipError_t launch_video_pad(const void* x, void* y, int dtype, int B, int C, int T, int H, int W, int t0, int nt,
                            int Tp, int Hp, int Wp, hipStream_t s) {
    const int planes = B * C * Tp;
    const WinGeom g = win_geom(T, H, W, t0, nt, Tp, Hp, Wp, planes);
    return dtype == CVT_F32 ? launch_pad_t<uint32_t>(x, y, planes, g, s) : launch_pad_t<uint16_t>(x, y, planes, g, s);
}

hipError_t launch_video_unpad(const void* y, void* x, int dtype, int B, int C, int T, int H, int W, int t0, int nt,
                              int Tp, int Hp, int Wp, hipStream_t s) {
    const int planes = B * C * nt;
    const WinGeom g = win_geom(T, H, W, t0, nt, Tp, Hp, Wp, planes);
    return dtype == CVT_F32 ? launch_unpad_t<uint32_t>(y, x, planes, g, s)
                            : launch_unpad_t<uint16_t>(y, x, planes, g, s);
}

}  // namespace cvt
