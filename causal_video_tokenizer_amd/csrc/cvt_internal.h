// Internal declarations shared by the HIP translation units of libcvt.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cvt.h"

namespace cvt {

// ---------------------------------------------------------------- device helpers

// bf16 is handled as raw 16-bit patterns; widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
}

// Swish y * sigmoid(y) with the hardware reciprocal (about 1 ulp) instead of a division.
__device__ __forceinline__ float swish_f(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

// Non-temporal (streaming) loads for data read exactly once: on gfx950 they raise
// the achievable read bandwidth of a streaming kernel noticeably over plain loads.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Streaming (non-temporal) stores for outputs that no later access of the same kernel reads.
__device__ __forceinline__ void st_stream8(void* p, uint2 v) {
    const u32x2_t t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// One window of a clip (sliding windows over a video of any length): frames t0 .. t0+nt-1
// of a T x H x W clip, seen as a padded window whose frame p is clip frame
// t0 + mirror_frame(p, nt) and whose rows >= H and columns >= W are zero.
struct ClipWindow {
    int T, H, W;  // the clip
    int t0, nt;   // the window's frames
};

// Padded frame t of an n-frame window: t itself inside the window, then the mirror about
// the last frame without repeating it, bouncing between the two ends (period 2(n-1)).
__device__ __forceinline__ int mirror_frame(int t, int n) {
    if (n == 1) return 0;
    const int p = 2 * (n - 1);
    const int m = t % p;
    return m < n ? m : p - m;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are already
// validated by the C ABI layer.

// win == nullptr: x is the whole [B, C, T, H, W] input.  Otherwise T, H, W are the padded
// window's sizes and the pixels come from (go to) the clip win describes.
hipError_t launch_haar_fwd(const void* x, int x_dtype, void* y, int y_dtype, int y_layout,
                           int B, int C, int T, int H, int W, int temporal_levels,
                           hipStream_t stream, const ClipWindow* win = nullptr);
hipError_t launch_haar_inv(const void* y, int y_dtype, int y_layout, void* x, int x_dtype,
                           int B, int C, int T, int H, int W, int temporal_levels,
                           hipStream_t stream, const ClipWindow* win = nullptr);

// FSQ parameters precomputed on the host (double precision) and passed by value.
constexpr int FSQ_MAX_D = 8;
constexpr int FSQ_MAX_L = 16;
struct FsqParams {
    int D;
    int nthr[FSQ_MAX_D];                    // L_i - 1 breakpoints per channel
    int half[FSQ_MAX_D];                    // floor(L_i / 2)
    int levels[FSQ_MAX_D];
    int basis[FSQ_MAX_D];                   // mixed-radix place values
    unsigned int magic[FSQ_MAX_D];          // floor(n / L_i) = mulhi(n, magic) >> shift, n < 2^31
    int shift[FSQ_MAX_D];
    float thr[FSQ_MAX_D][FSQ_MAX_L - 1];    // digit = #{j : z >= thr[i][j]}
    int codebook;                           // product of the levels
};

// Exact floor(n / L) for 0 <= n < 2^31 and 2 <= L <= 16.  With l = ceil(log2 L),
// M = ceil(2^(31+l) / L) < 2^32 and n M / 2^(31+l) exceeds n / L by less than
// n / 2^(31+l) < 2^-l <= 1/L, the smallest gap between n / L and the next
// integer, so floor(mulhi(n, M) / 2^(l-1)) = floor(n / L).
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t M, int sh) {
    return __umulhi(n, M) >> sh;
}

hipError_t launch_fsq_quantize(const void* z, int z_dtype, int z_layout, int32_t* idx, void* codes,
                               const FsqParams& p, long long B, long long npos_per_b,
                               hipStream_t stream);
hipError_t launch_fsq_dequantize(const int32_t* idx, void* codes, int c_dtype, int c_layout,
                                 const FsqParams& p, long long B, long long npos_per_b,
                                 int32_t* invalid, hipStream_t stream);

// Factorized causal convolution.
size_t conv_workspace_bytes(int B, int Cin, int Cout, int T, int H, int W, int k, bool spatial, bool temporal);
hipError_t launch_conv_fact(const void* x, const void* w_s, const void* w_t, const float* b_s,
                            const float* b_t, void* y, int B, int Cin, int Cout, int T, int H,
                            int W, int k, void* workspace, hipStream_t stream);
// cvt_causal_conv3d_fact with the library's preallocated scratch as the workspace
// (noalloc.hip); conv_workspace_bytes() must not exceed CVT_NOALLOC_SCRATCH_BYTES.
hipError_t launch_conv_fact_noalloc(const void* x, const void* w_s, const void* w_t, const float* b_s,
                                    const float* b_t, void* y, int B, int Cin, int Cout, int T, int H, int W, int k,
                                    hipStream_t stream);
// Cross-stage fusion (conv.hip): the factorized conv of the Haar coefficients of a 3-channel
// bf16 clip [B, 3, T, H, W] (pixel sizes; coefficients computed in the spatial conv's loads),
// and of the D -> Cmid projection of dequantized FSQ indices [B, T, H, W].
size_t haar_conv_workspace_bytes(int B, int Cout, int T, int H, int W, bool temporal);
hipError_t launch_haar_conv(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                            void* y, int B, int Cout, int T, int H, int W, void* workspace, hipStream_t s);
size_t fsq_conv_workspace_bytes(int B, int Cmid, int Cout, int T, int H, int W, bool temporal);
// Factorized causal convolution followed by a 1x1x1 projection to Cp channels.
size_t conv_proj_workspace_bytes(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k, bool spatial,
                                 bool temporal);
// With idx (and fsq), FSQ of the projected latent too: the indices are computed in the
// projection's epilogue where it is fused (y may then be nullptr), else by the FSQ kernel
// on the latent; the workspace is then conv_proj_fsq_workspace_bytes.
hipError_t launch_conv_fact_proj(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                                 const void* w_p, const float* b_p, void* y, int B, int Cin, int Cout, int Cp, int T,
                                 int H, int W, int k, void* workspace, hipStream_t s, int32_t* idx = nullptr,
                                 const FsqParams* fsq = nullptr);
size_t conv_proj_fsq_workspace_bytes(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k, bool spatial,
                                     bool temporal);
// FSQ dequantize followed by the 1x1 projection D -> Cout (the decoder's first layer), one
// kernel: y [positions][Cout] bf16 = w_p . bf16(codes) + b_p.
hipError_t launch_fsq_dequant_proj(const int32_t* idx, const FsqParams& p, const void* w_p, const float* b_p, void* y,
                                   long long P, int Cout, int32_t* invalid, hipStream_t s);
hipError_t launch_fsq_conv(const int32_t* idx, const FsqParams& p, const void* w_lift, const float* b_lift,
                           const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y, int B,
                           int Cmid, int Cout, int T, int H, int W, void* workspace, hipStream_t s);

// Weights packed once by the caller (conv.hip): the row-tiled kernels' fragment order
// (taps 9, 3 or 1), and the factorized conv (with the fused 1x1) on packed weights.
size_t conv_weights_packed_bytes(int Cout, int Cin, int taps);
hipError_t launch_conv_weights_pack(const void* w, void* packed, int Cout, int Cin, int taps, hipStream_t s);
bool conv_packed_supported(int Cin, int Cout, int H, int W, bool spatial, bool temporal);
size_t conv_packed_workspace_bytes(int B, int Cout, int T, int H, int W, bool spatial, bool temporal);
hipError_t launch_conv_fact_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s,
                                   const float* b_t, void* y, int B, int Cin, int Cout, int T, int H, int W,
                                   void* workspace, hipStream_t s);
bool conv_proj_packed_supported(int Cin, int Cout, int Cp, int H, int W, bool spatial);
size_t conv_proj_packed_workspace_bytes(int B, int Cout, int T, int H, int W, bool spatial);
hipError_t launch_conv_fact_proj_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s,
                                        const float* b_t, const void* pw_p, const float* b_p, void* y, int B, int Cin,
                                        int Cout, int Cp, int T, int H, int W, void* workspace, hipStream_t s);

// Causal temporal convolution of one chunk of a stream (conv.hip): history frames in place
// of the zero padding, optional fused 1x1 projection (C <= 256, Cp <= 16).
size_t conv_temporal_stream_workspace_bytes(int C, int Cp);
bool conv_temporal_stream_supported(int C, int Cp, long long HW);
hipError_t launch_conv_temporal_stream(const void* x, const void* hist, const void* w_t, const float* b_t,
                                       const void* w_p, const float* b_p, void* y, int B, int C, int Cp, int T,
                                       int H, int W, void* workspace, hipStream_t s);

// Factorized self-attention (attention.hip).  Spatial: head dim 64; temporal causal:
// head dim 32 or 64 and T * C <= attention_max_tc().
int attention_max_tc();
hipError_t launch_attention3d(const void* q, const void* k, const void* v, void* out, int B, int C, int T, int H,
                              int W, int heads, int axis, hipStream_t stream);

// Sliding-window padding and cropping (window.hip).  Arguments validated by the ABI layer:
// planes of Hp*Wp and H*W elements below 2^30, B*C*Tp below 2^31.
hipError_t launch_video_pad(const void* x, void* y, int dtype, int B, int C, int T, int H, int W, int t0, int nt,
                            int Tp, int Hp, int Wp, hipStream_t s);
hipError_t launch_video_unpad(const void* y, void* x, int dtype, int B, int C, int T, int H, int W, int t0, int nt,
                              int Tp, int Hp, int Wp, hipStream_t s);

// LayerNorm (+ Swish) over the channels of an NTHWC bf16 tensor (norm.hip); x == y allowed.
hipError_t launch_layernorm(const void* x, const float* gamma, const float* beta, void* y, long long P, int C,
                            float eps, int swish, hipStream_t s);

// Encoder / decoder blocks (conv.hip).
bool resblock_supported(int C, int H, int W);
size_t resblock_workspace_bytes(int B, int C, int T, int H, int W, bool packed = false);
hipError_t launch_resblock(const void* x, const cvt_resblock_weights& w, void* y, int B, int C, int T, int H, int W,
                           float eps, void* workspace, hipStream_t s, bool packed = false);
bool downsample_packed_supported(int Cin, int Cout, int H, int W, bool space, bool time);
size_t downsample_workspace_bytes(int B, int Cin, int Cout, int T, int H, int W, bool space, bool time,
                                  bool packed = false);
hipError_t launch_downsample(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                             void* y, int B, int Cin, int Cout, int T, int H, int W, void* workspace, hipStream_t s,
                             bool packed = false);
bool upsample_supported(int Cin, int Cout, int W_in, long long HW_mid);
size_t upsample_workspace_bytes(int B, int Cin, int Cout, int T, int H, int W, bool up_space, bool packed = false);
hipError_t launch_upsample(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                           int B, int Cin, int Cout, int T, int H, int W, bool up_space, bool up_time, void* workspace,
                           hipStream_t s, bool packed = false);

}  // namespace cvt
