// Factorized causal 3D convolution as bf16 MFMA implicit GEMMs.
//
// The operation is the one in "Cosmos World Foundation Model Platform for
// Physical AI (Cosmos-Predict1)", section "1) Cosmos Tokenizer": a 1 x k x k
// spatial convolution followed by a k x 1 x 1 temporal convolution whose k-1
// frames of left padding make it causal (the model card's "Model
// Architecture" calls these causal temporal convolutions).
//
// Each of the two convolutions is a GEMM over
//   M = output channels, N = positions (b, t, y, x), K = taps x input channels,
// with the activation operand gathered on the fly from the NTHWC tensor: for
// tap j the activation row of position (b, t, y, x) is the input row at
// (b, t + dt_j, y + dy_j, x + dx_j), or zeros outside the tensor.  Spatial taps
// are (0, dy - (k-1)/2, dx - (k-1)/2) for the k*k kernel entries; temporal
// taps are (j - (k-1), 0, 0), so frames before 0 read zeros (causal left
// padding) and no frame after t is ever read.
//
// Kernels:
//   * conv_rows_kernel - the hot path, k = 3 with Cout >= 64 and Cout % 8 == 0:
//     both parts as a 3-tap filter along a row axis (image rows or frames), R
//     output rows per workgroup sharing one staged input region, weights read
//     from L2 in MFMA fragment order (layout and schedule at the kernel);
//   * conv_igemm_kernel - every other shape (k = 1 projections, narrow outputs):
//     one tap x 64 input channels per K step, weight and activation tiles staged
//     in LDS with XOR-swizzled 128-byte rows, 4 waves of 32 x 32 MFMA blocks;
//   * pointwise_small_kernel - 1 x 1 x 1 with at most 16 input channels (fp32 FMA).
// All of them add the optional fp32 bias and round to bf16 (RNE) once.
#include <algorithm>
#include <type_traits>

#include "cvt_internal.h"

namespace cvt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;          // input channels per K step
constexpr int ROWB = BK * 2;    // bytes per LDS row

// Tap geometry of the GEMM's K dimension, fixed at compile time.
enum TapKind { SPATIAL3 = 0, TEMPORAL3 = 1, POINT = 2 };

template <int KIND>
struct Taps;
template <>
struct Taps<SPATIAL3> {  // 1 x 3 x 3, zero padding 1: tap = 3 * dy + dx
    static constexpr int n = 9;
    __device__ static int dt(int) { return 0; }
    __device__ static int dy(int j) { return j / 3 - 1; }
    __device__ static int dx(int j) { return j % 3 - 1; }
};
template <>
struct Taps<TEMPORAL3> {  // 3 x 1 x 1, causal: tap j reads frame t + j - 2
    static constexpr int n = 3;
    __device__ static int dt(int j) { return j - 2; }
    __device__ static int dy(int) { return 0; }
    __device__ static int dx(int) { return 0; }
};
template <>
struct Taps<POINT> {
    static constexpr int n = 1;
    __device__ static int dt(int) { return 0; }
    __device__ static int dy(int) { return 0; }
    __device__ static int dx(int) { return 0; }
};

struct ConvGeom {
    long long P;                // output positions = B*T*H*W
    int T, H, W;                // output grid
    int Cin, Cout;
    int kchunks;                // ceil(Cin / BK)
    // input grid and strides of conv_igemm_kernel (stride 2 = the downsampling convolution:
    // output (t, y, x) reads input (st t + dt, ss y + dy, ss x + dx)); st = 0 means the input
    // grid is the output grid at stride 1
    int Ti, Hi, Wi, st, ss;
    // conv_rows_kernel reading a nearest-neighbour upsampled input (x2 in H and W for the
    // spatial part, causal x2 in time for the temporal part): Ti, Hi, Wi are then the input's
    int ups;
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int KIND, int TC, int TP, int WC, int WP>
__global__ __launch_bounds__(256) void conv_igemm_kernel(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ Wp,
                                                         const float* __restrict__ bias,
                                                         uint16_t* __restrict__ Y, ConvGeom g) {
    static_assert(WC * WP == 4, "4 waves per workgroup");
    constexpr int WTC = TC / WC, WTP = TP / WP;      // wave sub-tile
    constexpr int FA = WTC / 32, FB = WTP / 32;      // 32x32 blocks per wave
    constexpr int LA = TC / 32, LB = TP / 32;        // 16-byte chunks loaded per thread
    static_assert(FA >= 1 && FB >= 1, "wave tile too small");

    __shared__ __attribute__((aligned(16))) uint8_t smem[(TC + TP) * ROWB];
    uint8_t* sA = smem;
    uint8_t* sB = smem + TC * ROWB;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wc = wave % WC, wp = wave / WC;

    const int ntc = (g.Cout + TC - 1) / TC;
    const long long tile = blockIdx.x;
    const int tc_idx = (int)(tile % ntc);
    const long long p0 = (tile / ntc) * TP;
    const int n0 = tc_idx * TC;

    // loader roles: chunk (8 channels) and row base
    const int chunk = tid & 7;
    const int rbase = tid >> 3;  // 0..31

    // decode the activation rows this thread loads: output (b, t, y, x) -> input base row
    // (b, st t, ss y, ss x)
    int bt_[LB], by_[LB], bx_[LB];
    long long bpos[LB];
    bool bin[LB];
    const long long HW = (long long)g.H * g.W;
    const long long HWi = (long long)g.Hi * g.Wi;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const long long pos = p0 + rbase + 32 * i;
        bin[i] = pos < g.P;
        const long long pc = bin[i] ? pos : 0;
        bx_[i] = (int)(pc % g.W) * g.ss;
        by_[i] = (int)((pc / g.W) % g.H) * g.ss;
        bt_[i] = (int)((pc / HW) % g.T) * g.st;
        const long long b = pc / (HW * g.T);
        bpos[i] = (b * g.Ti + bt_[i]) * HWi + (long long)by_[i] * g.Wi + bx_[i];
    }

    f32x16_t acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    using TP_ = Taps<KIND>;
    const int nsteps = TP_::n * g.kchunks;
    uint4 ra[LA], rb[LB];

    auto gload = [&](int tap, int kc) {
        const int c0 = kc * BK + chunk * 8;
        const bool cval = c0 < g.Cin;
        const int dt = TP_::dt(tap), dy = TP_::dy(tap), dx = TP_::dx(tap);
        const long long doff = (long long)dt * HWi + (long long)dy * g.Wi + dx;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            const int n = n0 + rbase + 32 * i;
            if (cval && n < g.Cout)
                ra[i] = *reinterpret_cast<const uint4*>(Wp + ((size_t)n * TP_::n + tap) * g.Cin + c0);
            else
                ra[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int t = bt_[i] + dt, y = by_[i] + dy, x = bx_[i] + dx;
            const bool v = cval && bin[i] && t >= 0 && t < g.Ti && y >= 0 && y < g.Hi && x >= 0 && x < g.Wi;
            if (v)
                rb[i] = *reinterpret_cast<const uint4*>(X + (size_t)(bpos[i] + doff) * g.Cin + c0);
            else
                rb[i] = make_uint4(0, 0, 0, 0);
        }
    };

    gload(0, 0);
    int ntap = 0, nkc = 0;  // (tap, channel step) of the next K step
    for (int step = 0; step < nsteps; ++step) {
        if (++nkc == g.kchunks) {
            nkc = 0;
            ++ntap;
        }
        __syncthreads();  // previous step's LDS reads are complete
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            const int row = rbase + 32 * i;
            *reinterpret_cast<uint4*>(sA + row * ROWB + swz(row, chunk) * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int row = rbase + 32 * i;
            *reinterpret_cast<uint4*>(sB + row * ROWB + swz(row, chunk) * 16) = rb[i];
        }
        __syncthreads();
        if (step + 1 < nsteps) gload(ntap, nkc);

#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + (lane >> 5);
            bf16x8_t fa[FA], fb[FB];
#pragma unroll
            for (int a = 0; a < FA; ++a) {
                const int row = wc * WTC + a * 32 + (lane & 31);
                fa[a] = *reinterpret_cast<const bf16x8_t*>(sA + row * ROWB + swz(row, ch) * 16);
            }
#pragma unroll
            for (int b = 0; b < FB; ++b) {
                const int row = wp * WTP + b * 32 + (lane & 31);
                fb[b] = *reinterpret_cast<const bf16x8_t*>(sB + row * ROWB + swz(row, ch) * 16);
            }
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int b = 0; b < FB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
    }

    // epilogue: D[i][j], j = lane % 32 (position), i = 8 (r / 4) + 4 (lane / 32) + r % 4 (channel)
    const bool vec_store = (g.Cout & 3) == 0;
#pragma unroll
    for (int b = 0; b < FB; ++b) {
        const long long pos = p0 + wp * WTP + b * 32 + (lane & 31);
        if (pos >= g.P) continue;
        uint16_t* yrow = Y + (size_t)pos * g.Cout;
#pragma unroll
        for (int a = 0; a < FA; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wc * WTC + a * 32 + 8 * q + 4 * (lane >> 5);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[a][b][4 * q + e];
                    if (bias && n + e < g.Cout) v[e] += bias[n + e];
                }
                if (vec_store && n + 3 < g.Cout) {
                    uint2 u;
                    u.x = pack_bf16x2(v[0], v[1]);
                    u.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(yrow + n) = u;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < g.Cout) yrow[n + e] = f32_to_bf16(v[e]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// 3-tap-set convolutions over R output rows per workgroup (the hot kernels).
//
// Both convolutions are a 3-tap filter along one "row" axis, repeated over KX column
// shifts:
//   TEMPORAL3: rows are frames, columns are NC flattened (h, w) positions; output frame t
//              reads input frames t-2, t-1, t through taps 0, 1, 2 (KX = 1);
//   SPATIAL3:  rows are image rows of one frame, columns are NC pixels of a row plus a
//              1-pixel halo (NC + 2); output row y, pixel x reads input row y-1+ky, pixel
//              x-1+kx through tap (ky, kx) (KX = 3).
// One workgroup (4 or 8 waves) computes TCH output channels x NC columns x R consecutive
// output rows r0 .. r0+R-1, which read the R+2 input rows r0-off .. r0+R-1 (off = 2
// temporal, 1 spatial): the REGION, staged once per BK-channel K chunk.  Region row rr
// meets tap row ky in output row r0 + rr - ky.  Each wave owns FA 32-channel x FB 32-column
// MFMA blocks (FA * FB = 2) over all R rows: per (16-channel k-step, column shift kx) it
// takes its 3 FA weight fragments (3 tap rows) once and walks the region rows, each
// activation fragment feeding up to three tap rows, i.e. three output rows.  Up to 256
// output channels both convolutions use 4 waves of FA = 2, FB = 1 (64 channels x 32
// columns per wave), so each region is staged once for every output channel and two
// workgroups share a CU; their six weight fragments per step are requested right after
// the previous use of their registers.  FA = 1, FB = 2 (32 x 64 per wave, half the weight
// bytes per MFMA) serves up to 128 channels, and the temporal conv above 256 channels
// (8 waves).  A step's activation reads are issued during the
// previous step's MFMAs (see compute), so only a chunk's first step waits for LDS.
//
// Only the region is staged in LDS (two buffers of 30-36 KB; two 4-wave workgroups share a
// CU, so one's barrier and epilogue overlap the other's MFMAs).  The weights are packed
// once per call in MFMA fragment order (see pack_frag_kernel): each fragment is 1 KB of
// which lane l reads bytes [16 l, 16 l + 16), one coalesced load straight into the operand
// registers, prefetched one step ahead.  The region loads of chunk c + 1 are issued in two
// batches during chunk c, each after that step's weight prefetch and stored a few steps
// later, so a weight wait never waits for a region load issued less than two steps before.
//
// Rows and columns outside the tensor read zeros (padding, including the causal frames
// before 0): every global load is a raw buffer load whose resource is sized to the tensor
// and padding rows get an offset past its end.  Output rows past the end are neither
// computed (the count of valid rows is a compile-time branch per tile) nor stored.
// Blocks are mapped to tiles XCD by XCD: block L runs tile (L mod 8) * per_xcd + L / 8,
// so consecutive tiles - the channel tiles of one region, then the row tiles above and
// below it, which re-read two of its rows - share an L2.
struct RowsGeom {
    int B, T, H, W, HW, Cin, Cout;
    long long x_total;      // bytes of the input tensor (any size: a tile's region is addressed from its own base)
    int wf_bytes;           // packed weights' buffer-resource extent
    int NA, KC16;           // 32-row weight blocks, 16-channel k-steps
    int nct, ncol, nrow;    // channel tiles, column tiles, row tiles
    int ntiles, per_xcd;
    int Cp, wp_bytes;       // fused 1x1 projection: output channels, packed weight bytes (0 = none)
    long long h_total;      // temporal stream: bytes of the two history frames [B][2][HW][Cin] (0 = none)
    int ups;                // input nearest-neighbour upsampled (spatial: x2 in H, W; temporal: causal x2)
    int Ti, Hi, Wi;         // with ups: the input grid
};

// Epilogues of conv_rows_kernel.  PLAIN: bias, bf16.  PROJ: the fused 1x1 projection.
// NORM: LayerNorm over the Cout channels of each position (scale, shift) and optionally
// Swish.  RES: a residual tensor shaped like the output added before the rounding.  PROJ
// and NORM need every output channel in the workgroup (one channel tile).
// PFSQ: PROJ followed by FSQ of the bf16 latent (indices out, the latent optional).
constexpr int EPI_PLAIN = 0, EPI_PROJ = 1, EPI_NORM = 2, EPI_RES = 3, EPI_PFSQ = 4;
template <int EPI>
constexpr bool epi_proj() {
    return EPI == EPI_PROJ || EPI == EPI_PFSQ;
}
struct RowsAux {
    const uint16_t* res;   // RES: [positions][Cout] bf16, the output's layout
    const float* ln_g;     // NORM: per-channel scale and shift, float32 [Cout]
    const float* ln_b;
    float eps;             // NORM: added to the variance
    int swish;             // NORM: apply Swish after the affine step
    int32_t* fsq_idx;      // PROJ: FSQ indices of the projected latent (nullptr = none)
    FsqParams fsq;         // PROJ with fsq_idx, and SRC_FSQ: the level set (D = Cp <= 8)
    int px_T;              // SRC_HAAR: frames of the pixel clip (4 T' - 3)
    const uint16_t* lift_w;  // SRC_FSQ: the projection D -> Cin, bf16 [Cin][D]
    const float* lift_b;     // SRC_FSQ: its bias, float32 [Cin] or nullptr
};

// LDS bytes per region row: BK channels + 16 bytes of padding
template <int BK>
constexpr int rows_xs() {
    return BK * 2 + 16;
}
constexpr int ROWS_OOB_BASE = 0x7fff0000;  // buffer offset base of padding rows (a tile's span stays below it)

// Tile configuration.  A workgroup has NW waves (3, 4 or 8): WCH along output channels and
// NW / WCH along columns.  Each wave owns FA 32-channel MFMA blocks x FB 32-column blocks
// (FA * FB = 2, so 128 fp32 accumulators for R = 4 rows) over all R output rows.
#ifndef CVT_ROWS_SP_PD
#define CVT_ROWS_SP_PD 1
#endif
// S = 2: the stride-2 (downsampling) convolution.  Output row i reads input rows S i + j
// (temporal: frames 2 (r0 + i) - 2 + j; spatial: rows 2 (r0 + i) - 1 + ky), so a tile of R
// output rows stages S (R - 1) + 3 input rows.  Spatially the 2 NC + 1 input columns of a
// tile are staged de-interleaved, the NC + 1 odd ones (input columns 2 c0 - 1 + 2 m) first
// and the NC even ones (2 c0 + 2 m) after them, so the column shifts kx = 0, 1, 2 read the
// contiguous runs starting at region columns 0, NC + 1 and 1.
// SRC: where the region's input channels come from.  SRC_TENSOR: the NTHWC input tensor.
// The other two compute them while staging (cross-stage fusion, spatial conv at stride 1 on
// 256-thread workgroups with one region row per thread):
//   SRC_HAAR: X holds the pixel clip [B, 3, 4T'-3, 4H, 4W] (bf16 NCTHW) and the 192 input
//     channels are its 2-level Haar coefficients in pixel-channel order (see haar_region);
//   SRC_FSQ: X holds int32 FSQ indices [B, T, H, W] and the input channels are the 1x1
//     projection of their dequantized codes (see fsq_region).
constexpr int SRC_TENSOR = 0, SRC_HAAR = 1, SRC_FSQ = 2;
constexpr int LIFT_MAX_C = 256;                          // SRC_FSQ: widest projection staged in LDS
constexpr int LIFT_BYTES = (FSQ_MAX_D + 1) * LIFT_MAX_C * 4;  // its weights [c][n] and bias, float32

template <int KIND_, int R_, int WCH_, int FA_, int BK_, int NW_ = 4, int S_ = 1, int SRC_ = SRC_TENSOR>
struct RowsCfg {
    static constexpr int KIND = KIND_, R = R_, WCH = WCH_, FA = FA_, FB = 2 / FA_, BK = BK_, NW = NW_, S = S_;
    static constexpr int SRC = SRC_;
    static constexpr int NTH = 64 * NW;                         // threads per workgroup
    static constexpr int WPOS = NW / WCH;                       // waves along columns
    static constexpr int KX = KIND == SPATIAL3 ? 3 : 1;         // column shifts
    static constexpr int TCH = 32 * FA * WCH;                   // output channels per workgroup
    static constexpr int NC = 32 * FB * WPOS;                   // output columns per workgroup
    static constexpr int RC = KIND == SPATIAL3 ? S * NC + (S == 1 ? 2 : 1) : NC;  // region columns (with the x halo)
    static constexpr int RROWS = S * (R - 1) + 3;                                  // region rows
    static constexpr int XS = rows_xs<BK>();
    // region rows per buffer, padded so that the 16-byte chunks (BK / 8 per row) split evenly
    // over the 256 threads: every thread issues the same unguarded loads (padding rows read
    // zeros and are never used), which keeps the compiler from sinking a guarded load into a
    // branch followed by a full memory wait
    static constexpr int PD = KIND == SPATIAL3 ? CVT_ROWS_SP_PD : 1;  // weight prefetch distance in steps
    static constexpr int PASS = NTH / (BK / 8);
    static constexpr int XROWS = (RROWS * RC + PASS - 1) / PASS * PASS;
    static constexpr int REGION_BYTES = 2 * XROWS * rows_xs<BK>();       // the two region buffers
    static constexpr int PRS = TCH * 2 + 16;                              // fused projection: bytes per staged column
    static constexpr int PROJ_BYTES = R * NC * PRS;                       // R frames of staged columns
    static constexpr int RES_BYTES = NW * 32 * FB * (128 * FA + 16);       // residual epilogue: float32 row stages
    static_assert((NW == 3 || NW == 4 || NW == 8) && WCH * WPOS == NW && FA * FB == 2 && (BK == 32 || BK == 64) && R >= 1 &&
                      R <= 4 && (S == 1 || S == 2),
                  "tile shape");
    static_assert(SRC == SRC_TENSOR || (KIND == SPATIAL3 && S == 1 && BK == 32 && RROWS * RC <= NTH && XROWS == NTH),
                  "computed regions: spatial, stride 1, 32-channel chunks, one region row per thread");
};

template <typename C, int NV, bool TAIL, int EPI, bool HIST>
__device__ __forceinline__ void rows_tile(const uint16_t* __restrict__ Wf, const uint16_t* __restrict__ X,
                                          const float* __restrict__ bias, uint16_t* __restrict__ Y,
                                          const uint16_t* __restrict__ Wpf, const float* __restrict__ bias_p,
                                          const uint16_t* __restrict__ Hx, const RowsGeom& g, const RowsAux& aux,
                                          uint8_t* smem, int b, int t, int ct, int r0, int c0) {
    constexpr int KIND = C::KIND, BK = C::BK, FA = C::FA, FB = C::FB;
    constexpr int NTH = C::NTH, RC = C::RC, KX = C::KX, CPR = BK / 8, XS = C::XS, KS = BK / 16;
    constexpr int WCH = C::WCH;
    constexpr int XROWS = C::XROWS;
    constexpr int XQ = XROWS * CPR;
    constexpr int XL = (XQ + NTH - 1) / NTH;
    constexpr int OOB = 0x7fffffff;
    constexpr int SR = C::S;
    constexpr int NRU = SR * (NV - 1) + 3;  // region rows that feed a valid output row
    static_assert(SR == 1 || !HIST, "stream history frames only at stride 1");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it in a scalar register
    const int wch = wave % WCH, wpos = wave / WCH;
    auto sX = [&](int buf) { return smem + buf * (XROWS * XS); };  // the two region buffers

    // Region chunk q of a thread is (row, c16) with 8 consecutive lanes on 8 consecutive rows
    // at one chunk: LDS stores go 8 lanes (128 bytes) at a time, and 8 rows of 80 bytes at
    // one offset cover 32 distinct banks, where 4 chunks of 2 rows would collide.
    auto xmap = [](int q, int& row, int& c16) {
        row = (q / (8 * CPR)) * 8 + (q & 7);
        c16 = (q >> 3) % CPR;
    };
    // The region is addressed from the tile's first input row (spatial: first image row of the
    // frame; temporal: first frame at the tile's first column), p0 positions into the tensor:
    // the buffer resource is based there, so the offsets below are tile-relative and the
    // tensor may have any size (the launcher keeps a tile's span below ROWS_OOB_BASE bytes).
    // Computed regions (SRC_HAAR, SRC_FSQ) address their smaller inputs from the start.
    const int ymin = KIND == SPATIAL3 ? max(SR * r0 - 1, 0) : 0;
    const int frmin = KIND == TEMPORAL3 ? max(SR * r0 - 2, 0) : 0;
    long long p0 = 0;
    if constexpr (C::SRC == SRC_TENSOR) {
        if (KIND == SPATIAL3 && SR == 2)
            p0 = ((long long)(b * g.T + t) * g.Hi + ymin) * g.Wi;
        else if (KIND == SPATIAL3)
            p0 = g.ups ? ((long long)(b * g.T + t) * g.Hi + (ymin >> 1)) * g.Wi : ((long long)(b * g.T + t) * g.H + ymin) * g.W;
        else if (SR == 2)
            p0 = ((long long)b * g.Ti + frmin) * g.HW + c0;
        else
            p0 = g.ups ? ((long long)b * g.Ti + ((frmin + 1) >> 1)) * g.HW + c0 : ((long long)b * g.T + frmin) * g.HW + c0;
    }
    int xbase[XL];
    int hbase[HIST ? XL : 1];  // HIST (temporal stream, first row tile): offsets into the history frames
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int q = tid + NTH * i;
        int row, c16;
        xmap(q, row, c16);
        const int rr = row / RC, cc = row % RC;
        bool ok = q < XQ && rr < NRU;
        int rel = 0;  // input position relative to p0
        if (KIND == SPATIAL3 && SR == 2) {  // stride 2: rows 2 r0 - 1 + rr, de-interleaved columns
            constexpr int NC = C::NC;
            const int y = 2 * r0 - 1 + rr;
            const int x = cc <= NC ? 2 * c0 - 1 + 2 * cc : 2 * c0 + 2 * (cc - NC - 1);
            ok = ok && y >= 0 && y < g.Hi && x >= 0 && x < g.Wi;
            rel = (y - ymin) * g.Wi + x;
        } else if (KIND == SPATIAL3) {
            const int y = r0 - 1 + rr, x = c0 - 1 + cc;
            ok = ok && y >= 0 && y < g.H && x >= 0 && x < g.W;
            rel = g.ups ? ((y >> 1) - (ymin >> 1)) * g.Wi + (x >> 1) : (y - ymin) * g.W + x;
        } else if (SR == 2) {  // stride 2: input frames 2 r0 - 2 + rr
            const int fr = 2 * r0 - 2 + rr, hw = c0 + cc;
            ok = ok && fr >= 0 && fr < g.Ti && hw < g.HW;
            rel = (fr - frmin) * g.HW + cc;
        } else {
            const int fr = r0 - 2 + rr, hw = c0 + cc;
            if constexpr (HIST) {  // frames -2 and -1 are the history frames 0 and 1 (based at the tile's column)
                const bool hok = ok && fr < 0 && hw < g.HW;
                hbase[i] = hok ? (((fr + 2) * g.HW + cc) * g.Cin + c16 * 8) * 2 : ROWS_OOB_BASE;
            }
            ok = ok && fr >= 0 && fr < g.T && hw < g.HW;
            // upsampled in time: output frame fr of the causal repetition is input frame (fr + 1) / 2
            rel = g.ups ? (((fr + 1) >> 1) - ((frmin + 1) >> 1)) * g.HW + cc : (fr - frmin) * g.HW + cc;
        }
        // rows outside the tensor get a base past its end for every chunk (chunk offsets stay
        // below 64 KiB)
        xbase[i] = ok ? (rel * g.Cin + c16 * 8) * 2 : ROWS_OOB_BASE;
    }
    const long long xoff = p0 * g.Cin;  // elements
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + xoff), (short)0, (int)min(g.x_total - 2 * xoff, (long long)ROWS_OOB_BASE), 0x00020000);
    const long long hoff64 = HIST ? ((long long)b * 2 * g.HW + c0) * g.Cin : 0;
    const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(HIST ? Hx + hoff64 : X), (short)0, HIST ? (int)min(g.h_total - 2 * hoff64, (long long)ROWS_OOB_BASE) : 0,
        0x00020000);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)Wf, (short)0, g.wf_bytes, 0x00020000);

    // The region of chunk c + 1 goes to the buffer last read in chunk c - 1, free since that
    // chunk's closing barrier, so it is loaded and stored in two batches inside chunk c
    // (batch 0: loads i < XH, batch 1: the rest), which halves the staging registers.  With
    // fewer than 4 steps per chunk there is one batch of all XL loads.
    constexpr int NS = KS * KX;                       // steps per chunk: (k-step, column shift)
    constexpr int XH = NS >= 4 ? (XL + 1) / 2 : XL;  // loads of batch 0 (short chunks: one batch)
    uint4 xr[XH];
    auto load_region_t = [&](int kc, int half) {  // kc past the last chunk reads zeros
#pragma unroll
        for (int i = half * XH; i < (half ? XL : XH); ++i) {
            int off = xbase[i] + kc * BK * 2;
            bool inc = true;  // chunk channels below Cin
            if (TAIL) {       // Cin not a multiple of BK: chunks past Cin read zeros
                int row, c16;
                xmap(tid + NTH * i, row, c16);
                inc = kc * BK + c16 * 8 < g.Cin;
                off = inc ? off : OOB;
            }
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0);
            uint4 u = *reinterpret_cast<const uint4*>(&v);
            if constexpr (HIST) {  // each row is in exactly one of the two buffers: the other reads zeros
                const int hoff = inc ? hbase[i] + kc * BK * 2 : OOB;
                const auto vh = __builtin_amdgcn_raw_buffer_load_b128(hres, hoff, 0, 0);
                const uint4 w = *reinterpret_cast<const uint4*>(&vh);
                u.x |= w.x; u.y |= w.y; u.z |= w.z; u.w |= w.w;
            }
            xr[i - half * XH] = u;
        }
    };
    auto store_region_t = [&](int buf, int half) {
#pragma unroll
        for (int i = half * XH; i < (half ? XL : XH); ++i) {
            const int q = tid + NTH * i;
            int row, c16;
            xmap(q, row, c16);
            if (XQ % NTH == 0 || q < XQ) *reinterpret_cast<uint4*>(sX(buf) + row * XS + c16 * 16) = xr[i - half * XH];
        }
    };

    // ---- computed regions: thread tid stages region row tid (region row prr, column pcc, i.e.
    // latent row py and column pxx of frame t), zeros outside the grid
    constexpr int SRC = C::SRC;
    const int prr = tid / RC, pcc = tid % RC;
    const int py = r0 - 1 + prr, pxx = c0 - 1 + pcc;
    const bool pok = tid < C::RROWS * RC && prr < NRU && py >= 0 && py < g.H && pxx >= 0 && pxx < g.W;
    // SRC_HAAR.  Chunk kc holds 32 coefficients of pixel channel kc / 2: those of level-1
    // temporal band q = kc % 2 (packet rows rt = 2 q, 2 q + 1), channel m = 16 (rt % 2) + 4 rh +
    // rw (pack_frag_kernel orders the weights to match).  By linearity the two temporal rows
    // of the 4-frame block are 2D transforms of A = P + Q and B = P - Q with P = f0 + s f1,
    // Q = f2 + s f3, s = (-1)^q; the two frame pairs are loaded in the two region batches,
    // and P waits in the thread's own (still free) region row between them.
    const int hrow = 8 * g.W;                 // bytes per pixel row
    const int hplane = 32 * g.H * g.W;        // bytes per pixel frame
    int hoff = 0;                             // the block's first row in frame 0 of pixel channel 0
    int hfr[4] = {0, 0, 0, 0};                // frame offsets: padded frame 4 t + f is frame max(4 t + f - 3, 0)
    if constexpr (SRC == SRC_HAAR) {
        hoff = b * 3 * aux.px_T * hplane + 4 * py * hrow + 8 * pxx;
#pragma unroll
        for (int f = 0; f < 4; ++f) hfr[f] = max(4 * t + f - 3, 0) * hplane;
    }
    uint2 hr[SRC == SRC_HAAR ? 8 : 1];        // 4 rows of 4 pixels of two frames
    auto haar_load = [&](int kc, int half) {  // kc past the last chunk reads zeros
        const bool ok = pok && kc * BK < g.Cin;
        const int cbase = hoff + (kc >> 1) * aux.px_T * hplane;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int off = ok ? cbase + hfr[2 * half + f] + r * hrow : OOB;
                hr[4 * f + r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(xres, off, 0, 0));
            }
    };
    auto pix = [](const uint2 u, int k) {
        return k == 0 ? bf16_lo(u.x) : k == 1 ? bf16_hi(u.x) : k == 2 ? bf16_lo(u.y) : bf16_hi(u.y);
    };
    auto haar_store = [&](int buf, int half, int kc) {
        float* rowf = reinterpret_cast<float*>(sX(buf) + tid * XS);
        const float sg = (kc & 1) ? -1.0f : 1.0f;
        if (half == 0) {  // P, parked in the row
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<float4*>(rowf + 4 * r) =
                    make_float4(pix(hr[r], 0) + sg * pix(hr[4 + r], 0), pix(hr[r], 1) + sg * pix(hr[4 + r], 1),
                                pix(hr[r], 2) + sg * pix(hr[4 + r], 2), pix(hr[r], 3) + sg * pix(hr[4 + r], 3));
            return;
        }
        float A[4][4], Bq[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 pv = *reinterpret_cast<const float4*>(rowf + 4 * r);
            const float P[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float Q = pix(hr[r], k) + sg * pix(hr[4 + r], k);
                A[r][k] = P[k] + Q;
                Bq[r][k] = P[k] - Q;
            }
        }
        auto packet = [](float& a, float& b, float& c, float& d) {  // rows 1/2 (1,1,1,1), (1,1,-1,-1), (1,-1,1,-1), (1,-1,-1,1), unscaled
            const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
            a = s0 + s1;
            b = s0 - s1;
            c = d0 + d1;
            d = d0 - d1;
        };
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            packet(A[r][0], A[r][1], A[r][2], A[r][3]);
            packet(Bq[r][0], Bq[r][1], Bq[r][2], Bq[r][3]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            packet(A[0][k], A[1][k], A[2][k], A[3][k]);
            packet(Bq[0][k], Bq[1][k], Bq[2][k], Bq[3][k]);
        }
        uint4* rowv = reinterpret_cast<uint4*>(rowf);
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // channels 8 j .. 8 j + 7: rh = 2 j, 2 j + 1 of A; then of B
            rowv[j] = make_uint4(pack_bf16x2(A[2 * j][0] * 0.125f, A[2 * j][1] * 0.125f),
                                 pack_bf16x2(A[2 * j][2] * 0.125f, A[2 * j][3] * 0.125f),
                                 pack_bf16x2(A[2 * j + 1][0] * 0.125f, A[2 * j + 1][1] * 0.125f),
                                 pack_bf16x2(A[2 * j + 1][2] * 0.125f, A[2 * j + 1][3] * 0.125f));
            rowv[2 + j] = make_uint4(pack_bf16x2(Bq[2 * j][0] * 0.125f, Bq[2 * j][1] * 0.125f),
                                     pack_bf16x2(Bq[2 * j][2] * 0.125f, Bq[2 * j][3] * 0.125f),
                                     pack_bf16x2(Bq[2 * j + 1][0] * 0.125f, Bq[2 * j + 1][1] * 0.125f),
                                     pack_bf16x2(Bq[2 * j + 1][2] * 0.125f, Bq[2 * j + 1][3] * 0.125f));
        }
    };
    // SRC_FSQ.  The position's index, the same for every chunk, is loaded once; chunk kc holds
    // output channels 32 kc .. 32 kc + 31 of the projection, each accumulated as the
    // dequantize + 1x1 kernel does (bias, then fmaf over the bf16-rounded codes in channel
    // order), so the staged values equal that kernel's bf16 output.  The projection weights
    // and bias sit in LDS after the region buffers as float32 [c][LIFT_MAX_C] rows (row
    // FSQ_MAX_D: the bias), read as broadcasts.
    int fidx = 0;
    if constexpr (SRC == SRC_FSQ) {
        const int pos = ((b * g.T + t) * g.H + py) * g.W + pxx;
        fidx = (int)__builtin_amdgcn_raw_buffer_load_b32(xres, pok ? pos * 4 : OOB, 0, 0);
    }
    auto fsq_store = [&](int buf, int kc) {
        const float* wl = reinterpret_cast<const float*>(smem + C::REGION_BYTES);
        const FsqParams& fp = aux.fsq;
        const bool bad = fidx < 0 || fidx >= fp.codebook;
        uint32_t rem = bad ? 0u : (uint32_t)fidx;
        float xv[FSQ_MAX_D];
        // the default level set (8, 8, 8, 5, 5, 5): bit fields and exact multiply-shift divisions
        // (q / 5 = (q * 205) >> 10 for q < 1024), the digits the general split gives
        const bool def = fp.D == 6 && fp.levels[0] == 8 && fp.levels[1] == 8 && fp.levels[2] == 8 &&
                         fp.levels[3] == 5 && fp.levels[4] == 5 && fp.levels[5] == 5;
        if (def) {
            const uint32_t q = rem >> 9, q5 = (q * 205u) >> 10, q25 = (q5 * 205u) >> 10;
            const int d[6] = {(int)(rem & 7u), (int)((rem >> 3) & 7u), (int)((rem >> 6) & 7u), (int)(q - 5u * q5),
                              (int)(q5 - 5u * q25), (int)q25};
#pragma unroll
            for (int i = 0; i < FSQ_MAX_D; ++i) {
                const float code = i < 3 ? (float)(d[i] - 4) * 0.25f : (float)(d[i < 6 ? i : 5] - 2) * 0.5f;
                xv[i] = i < 6 ? (bad ? __builtin_nanf("") : bf16_to_f32(f32_to_bf16(code))) : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < FSQ_MAX_D; ++i) {
            if (def) break;
            xv[i] = 0.0f;
            if (i < fp.D) {
                const uint32_t q = div_magic(rem, fp.magic[i], fp.shift[i]);
                const int d = (int)(rem - q * (uint32_t)fp.levels[i]);
                rem = q;
                const int h = fp.half[i];
                const float code = (h & (h - 1)) == 0 ? (float)(d - h) * (1.0f / (float)h) : (float)(d - h) / (float)h;
                xv[i] = bad ? __builtin_nanf("") : bf16_to_f32(f32_to_bf16(code));
            }
        }
        uint4* rowv = reinterpret_cast<uint4*>(sX(buf) + tid * XS);
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // 8 channels at a time
            const int n0 = kc * BK + 8 * j;
            float o[8];
            const float4 b0 = *reinterpret_cast<const float4*>(wl + FSQ_MAX_D * LIFT_MAX_C + n0);
            const float4 b1 = *reinterpret_cast<const float4*>(wl + FSQ_MAX_D * LIFT_MAX_C + n0 + 4);
            o[0] = b0.x; o[1] = b0.y; o[2] = b0.z; o[3] = b0.w; o[4] = b1.x; o[5] = b1.y; o[6] = b1.z; o[7] = b1.w;
#pragma unroll
            for (int c = 0; c < FSQ_MAX_D; ++c) {
                if (c < fp.D) {
                    const float4 w0 = *reinterpret_cast<const float4*>(wl + c * LIFT_MAX_C + n0);
                    const float4 w1 = *reinterpret_cast<const float4*>(wl + c * LIFT_MAX_C + n0 + 4);
                    o[0] = fmaf(w0.x, xv[c], o[0]); o[1] = fmaf(w0.y, xv[c], o[1]);
                    o[2] = fmaf(w0.z, xv[c], o[2]); o[3] = fmaf(w0.w, xv[c], o[3]);
                    o[4] = fmaf(w1.x, xv[c], o[4]); o[5] = fmaf(w1.y, xv[c], o[5]);
                    o[6] = fmaf(w1.z, xv[c], o[6]); o[7] = fmaf(w1.w, xv[c], o[7]);
                }
            }
            rowv[j] = pok ? make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                       pack_bf16x2(o[6], o[7]))
                          : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    if constexpr (SRC == SRC_FSQ) {  // the projection table, once per tile
        float* wl = reinterpret_cast<float*>(smem + C::REGION_BYTES);
        const int D = aux.fsq.D;
        for (int i = tid; i < (FSQ_MAX_D + 1) * LIFT_MAX_C; i += NTH) {
            const int c = i / LIFT_MAX_C, n = i - c * LIFT_MAX_C;
            float v = 0.0f;
            if (n < g.Cin) {
                if (c < D) v = bf16_to_f32(aux.lift_w[n * D + c]);
                else if (c == FSQ_MAX_D && aux.lift_b) v = aux.lift_b[n];
            }
            wl[i] = v;
        }
        __syncthreads();
    }
    // region batch `half` of chunk kc: loads, then (a few steps later) the LDS stores
    auto load_region = [&](int kc, int half) {
        if constexpr (SRC == SRC_TENSOR) load_region_t(kc, half);
        else if constexpr (SRC == SRC_HAAR) haar_load(kc, half);
    };
    auto store_region = [&](int buf, int half, int kc) {
        if constexpr (SRC == SRC_TENSOR) store_region_t(buf, half);
        else if constexpr (SRC == SRC_HAAR) haar_store(buf, half, kc);
        else if (half == 1) fsq_store(buf, kc);
    };

    // weight fragments of (k-step kc16, column shift kx): tap rows 0..2 of blocks ab0 ..
    // ab0 + FA - 1
    const int ab0 = ct * (FA * WCH) + wch * FA;
    // weight fragments are prefetched PD steps ahead into NSET = PD + 1 register sets; a
    // chunk's step count is a multiple of NSET, so step st of every chunk uses set st % NSET
    constexpr int PD = C::PD, NSET = PD + 1;
    static_assert(C::KX * KS % NSET == 0, "whole fragment-set cycles per chunk");
    bf16x8_t fa[NSET][3][FA];
    const int lane16 = lane * 16;
    auto load_frags_ky = [&](int kc16, int kx, int set, int ky) {
#pragma unroll
            for (int a = 0; a < FA; ++a) {
                const int ab = ab0 + a, tap = ky * KX + kx;
                // wave-uniform fragment base (scalar) plus the lane's 16 bytes.  Blocks past Cout
                // only feed outputs that are not stored, and k-steps past the last one are only
                // the never-used prefetch after the final step, so both are clamped to a valid
                // fragment (no select: a select here becomes a branch with a full memory wait).
                // With a channel tail (TAIL) the padded k-step must multiply zeros, so it reads
                // zeros past the buffer instead.
                const int abc = min(ab, g.NA - 1);
                int fbase;
                if (TAIL)
                    fbase = kc16 < g.KC16 ? ((kc16 * 3 * KX + tap) * g.NA + abc) * 1024 : OOB - 1024;
                else
                    fbase = ((min(kc16, g.KC16 - 1) * 3 * KX + tap) * g.NA + abc) * 1024;
                const int off = fbase + lane16;
                fa[set][ky][a] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, 0));
            }
    };
    auto load_frags = [&](int kc16, int kx, int set) {
#pragma unroll
        for (int ky = 0; ky < 3; ++ky) load_frags_ky(kc16, kx, set, ky);
    };

    f32x16_t acc[NV][FA][FB];
#pragma unroll
    for (int f = 0; f < NV; ++f)
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int cb = 0; cb < FB; ++cb)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[f][a][cb][e] = 0.0f;

    const int khalf = lane >> 5, px = lane & 31;
    // Activation fragments of step s, region row rr: FB 32-column blocks at column shift
    // s % KX, channels of k-step s / KX.
    auto read_row = [&](bf16x8_t (&f)[NRU][FB], const uint8_t* xb, int s, int rr) {
        const int ch = (s / KX) * 2 + khalf, kx = s % KX;
        // column shift kx starts at region column kx (stride 1) or, de-interleaved at stride 2,
        // at 0 (odd columns), NC + 1 (even columns) or 1 (odd columns, one further)
        const int kc0 = SR == 1 ? kx : (kx == 1 ? C::NC + 1 : kx / 2);
#pragma unroll
        for (int cb = 0; cb < FB; ++cb)
            f[rr][cb] = *reinterpret_cast<const bf16x8_t*>(xb + (rr * RC + cb * 32 + kc0) * XS + ch * 16);
    };
    // The MFMAs of region row rr: it meets tap row ky in output row (rr - ky) / S.
    auto mfma_row = [&](const bf16x8_t (&f)[NRU][FB], int set, int rr) {
#pragma unroll
        for (int ky = 0; ky < 3; ++ky) {
            const int d = rr - ky;
            if (d < 0 || d % SR != 0) continue;
            const int ry = d / SR;
            if (ry >= NV) continue;
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int cb = 0; cb < FB; ++cb)
                    acc[ry][a][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][ky][a], f[rr][cb], acc[ry][a][cb],
                                                                             0, 0, 0);
        }
    };
    // One step's MFMAs with the next step's activation reads software-pipelined into them:
    // row rr of step s + 1 is read right after the MFMAs of row rr of step s, the last use
    // of that row's registers, so every read has the rest of the step to arrive (the
    // scheduling barriers keep that order; left alone the compiler would move the reads).
    // Tiles of two 32-channel blocks per wave (one weight fragment per 4 MFMAs or fewer) with two
    // fragment sets (EARLY): tap row ky of a set is last used by region row ky + NRU - 3, so its
    // fragments for the step after next are requested right there (refill(ky)) instead of at the
    // start of the next step: a third more time for the L2 fetch, with no further registers.
    // (On the one-block spatial tiles, whose fragments feed twice as many MFMAs, it is slower.)
    constexpr bool EARLY = NSET == 2 && FA == 2;
    auto compute = [&](const bf16x8_t (&cur)[NRU][FB], bf16x8_t (&nxt)[NRU][FB], const uint8_t* xb, int s, int set,
                       bool read_next, auto refill) {
#pragma unroll
        for (int rr = 0; rr < NRU; ++rr) {
            mfma_row(cur, set, rr);
            if (read_next) read_row(nxt, xb, s + 1, rr);
            if constexpr (EARLY) {
                if (rr >= NRU - 3) refill(rr - (NRU - 3));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Steps of a chunk: the weight prefetch of step s + PD comes first, then the region
    // batches: batch 0 is loaded at step 0 and stored at step L1, batch 1 loaded at step L1
    // and stored at the chunk's end (with fewer than 4 steps both are loaded at step 0 and
    // stored at the end).  The memory counter completes in order, so a weight wait at step s
    // also waits for every region batch issued before step s - PD: with PD = 2 a region
    // load has at least three steps to arrive from HBM before any weight wait covers it.
    constexpr int L1 = NS >= 4 ? NS / 2 : 0;
    static_assert(L1 > 0 || XH == XL, "a single batch when both would be in flight together");
    const int nchunks = (g.Cin + BK - 1) / BK;
    // step s of chunk kc: k-step KS kc + s / KX, column shift s % KX (s >= NS: next chunk)
    auto prefetch = [&](int kc, int s) {
        const int kcs = s < NS ? kc : kc + 1, ss = s < NS ? s : s - NS;
        load_frags(KS * kcs + ss / KX, ss % KX, s % NSET);
    };
    auto prefetch_ky = [&](int kc, int s, int ky) {
        const int kcs = s < NS ? kc : kc + 1, ss = s < NS ? s : s - NS;
        load_frags_ky(KS * kcs + ss / KX, ss % KX, s % NSET, ky);
    };
#pragma unroll
    for (int s = 0; s < (EARLY ? NSET : PD); ++s) prefetch(0, s);
    load_region(0, 0);
    store_region(0, 0, 0);
    if (L1 > 0) {
        load_region(0, 1);
        store_region(0, 1, 0);
    }
    __syncthreads();
    bf16x8_t fb[2][NRU][FB];  // activation fragments of the current and the next step
    for (int kc = 0; kc < nchunks; ++kc) {
        const uint8_t* xb = sX(kc & 1) + (wpos * 32 * FB + px) * XS;
        const int nbuf = (kc + 1) & 1;
        // a chunk's first step reads its rows after the barrier (the other steps' rows are
        // read during the step before)
#pragma unroll
        for (int rr = 0; rr < NRU; ++rr) read_row(fb[0], xb, 0, rr);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if constexpr (!EARLY) prefetch(kc, st + PD);
            __builtin_amdgcn_sched_barrier(0);  // weight prefetch before any region load
            if (L1 > 0 && st == L1) store_region(nbuf, 0, kc + 1);
            if (st == 0) load_region(kc + 1, 0);
            if (L1 > 0 && st == L1) load_region(kc + 1, 1);
            // keep the prefetches issued here: left alone the scheduler sinks them towards
            // their use to save registers, which exposes the memory latency
            __builtin_amdgcn_sched_barrier(0);
            compute(fb[st & 1], fb[(st + 1) & 1], xb, st, st % NSET, st + 1 < NS,
                    [&](int ky) { prefetch_ky(kc, st + 2, ky); });
        }
        if (L1 == 0)
            store_region(nbuf, 0, kc + 1);
        else
            store_region(nbuf, 1, kc + 1);
        __syncthreads();
    }

    // ---- epilogue.  Bias of the accumulator elements: element 4 q + e of block a is output
    // channel (ab0 + a) * 32 + 8 q + 4 khalf + e.
    float bv[FA][4][4];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = (ab0 + a) * 32 + 8 * q + 4 * khalf + e;
                bv[a][q][e] = bias ? bias[min(n, g.Cout - 1)] : 0.0f;
            }

    if constexpr (epi_proj<EPI>()) {
        // Epilogues over whole position rows (temporal kernel with every output channel in the
        // workgroup).  The tile's conv outputs, bias added and rounded to bf16 once (what a
        // separate pass would read), are staged in LDS as [frame][column][channel] rows, and
        // each wave then takes (frame, 32-column block) pairs.  Channels past Cout are staged
        // as zeros.
        // PROJ: the projection weights (A operand, rows o < Cp, standard fragment order) times
        // the staged columns over all TCH channels (B operand), so every projected value is one
        // MFMA accumulation chain and no partial sums cross waves.
        constexpr int TCH = C::TCH, NC = C::NC, PRS = C::PRS, KST = TCH / 16;
        // the projection weights (the only 32-row block, Cp <= 32; k-steps past Cout read
        // zeros) are requested first and arrive while the tile is staged
        bf16x8_t fp[epi_proj<EPI>() ? KST : 1];
        if constexpr (epi_proj<EPI>()) {
            const __amdgpu_buffer_rsrc_t pres =
                __builtin_amdgcn_make_buffer_rsrc((void*)Wpf, (short)0, g.wp_bytes, 0x00020000);
#pragma unroll
            for (int ks = 0; ks < KST; ++ks)
                fp[ks] = __builtin_bit_cast(bf16x8_t,
                                            __builtin_amdgcn_raw_buffer_load_b128(pres, (ks * 64 + lane) * 16, 0, 0));
        }
#pragma unroll
        for (int ry = 0; ry < NV; ++ry)
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int cb = 0; cb < FB; ++cb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x16_t& c = acc[ry][a][cb];
                        const int n = (ab0 + a) * 32 + 8 * q + 4 * khalf;  // first of 4 channels (Cout % 8 == 0)
                        uint2 u;
                        u.x = pack_bf16x2(c[4 * q] + bv[a][q][0], c[4 * q + 1] + bv[a][q][1]);
                        u.y = pack_bf16x2(c[4 * q + 2] + bv[a][q][2], c[4 * q + 3] + bv[a][q][3]);
                        if (n >= g.Cout) u = make_uint2(0u, 0u);
                        *reinterpret_cast<uint2*>(smem + (ry * NC + wpos * 32 * FB + cb * 32 + px) * PRS + n * 2) = u;
                    }
        __syncthreads();
        const int Cp = g.Cp;
        float bp[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int o = 8 * (r / 4) + 4 * khalf + (r % 4);
            bp[r] = bias_p && o < Cp ? bias_p[o] : 0.0f;
        }
        constexpr int NBLK = NC / 32;  // 32-column blocks per frame
        for (int pr = wave; pr < NV * NBLK; pr += C::NW) {  // wave-uniform
            const int fr = pr / NBLK, cblk = pr % NBLK;
            const uint8_t* brow = smem + (fr * NC + cblk * 32 + px) * PRS + khalf * 16;
            f32x16_t pacc;
#pragma unroll
            for (int e = 0; e < 16; ++e) pacc[e] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KST; ++ks)
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp[ks], *reinterpret_cast<const bf16x8_t*>(brow + ks * 32),
                                                               pacc, 0, 0, 0);
            // element r < 8 is projection output 8 (r / 4) + 4 khalf + r % 4 at column px
            const int hw = c0 + cblk * 32 + px;
            if constexpr (EPI == EPI_PFSQ) {  // FSQ of the bf16 latent: lane khalf = 0 gathers outputs 4..7 from lane + 32
                float lat[4], up[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lat[r] = bf16_to_f32(f32_to_bf16(pacc[r] + bp[r]));
                    up[r] = __shfl_xor(lat[r], 32);
                }
                if (khalf == 0 && hw < g.HW) {
                    const float z[8] = {lat[0], lat[1], lat[2], lat[3], up[0], up[1], up[2], up[3]};
                    int acc = 0;
                    bool nan = false;
#pragma unroll
                    for (int i = 0; i < FSQ_MAX_D; ++i) {
                        if (i < aux.fsq.D) {
                            int d = 0;
#pragma unroll
                            for (int j = 0; j < FSQ_MAX_L - 1; ++j) {
                                if (j >= aux.fsq.nthr[i]) break;  // uniform: the channel's breakpoint count
                                d += (z[i] >= aux.fsq.thr[i][j]) ? 1 : 0;
                            }
                            acc += d * aux.fsq.basis[i];
                            nan |= z[i] != z[i];
                        }
                    }
                    aux.fsq_idx[((long long)b * g.T + r0 + fr) * g.HW + hw] = nan ? -1 : acc;
                }
            }
            if ((EPI != EPI_PFSQ || Y) && hw < g.HW) {
                uint16_t* yp = Y + (((long long)b * g.T + r0 + fr) * g.HW + hw) * Cp;
                if ((Cp & 3) == 0) {  // 4 consecutive outputs per 8-byte store
#pragma unroll
                    for (int hq = 0; hq < 2; ++hq) {
                        const int o = 8 * hq + 4 * khalf;
                        if (o < Cp) {
                            uint2 u;
                            u.x = pack_bf16x2(pacc[4 * hq] + bp[4 * hq], pacc[4 * hq + 1] + bp[4 * hq + 1]);
                            u.y = pack_bf16x2(pacc[4 * hq + 2] + bp[4 * hq + 2], pacc[4 * hq + 3] + bp[4 * hq + 3]);
                            *reinterpret_cast<uint2*>(yp + o) = u;
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int o = 8 * (r / 4) + 4 * khalf + (r % 4);
                        if (o < Cp) yp[o] = f32_to_bf16(pacc[r] + bp[r]);
                    }
                }
            }
        }
        return;
    }

    // Bias, bf16 RNE, staged per output row through a wave-private LDS tile of 32 FB columns
    // x 32 FA channels (rows of 64 FA bytes + 16 bytes of padding, so the 8-byte writes of 8
    // consecutive columns hit distinct banks), then written back with each 4 FA consecutive
    // lanes storing one position's 64 FA contiguous bytes, as streaming (non-temporal) stores:
    // the output is not read again by this kernel (identical output; 1.8-2.3% faster than plain
    // stores per 720p layer, 0.3-0.8% over a chain of layers, whose next layer reads it).  The region buffers are free after
    // the last barrier of the K loop; a wave reads back only what it wrote and its LDS
    // accesses execute in order, so no barrier is needed.
    // RES stages the float32 sums instead (rows of 128 FA + 16 bytes) and adds the residual in
    // the store step, where each lane's 16 residual bytes sit at its store's offset (one
    // coalesced load per store, all of the tile's requested before the first staging) before
    // the single bf16 rounding.  A wave reads only the residual chunks it overwrites itself, each
    // before its store, so the output may be the residual tensor.
    constexpr int ES = EPI == EPI_RES ? 4 : 2;  // staged element bytes
    constexpr int OS = 32 * FA * ES + 16;
    constexpr int STAGE = 32 * FB * OS;  // bytes per wave
    static_assert(C::NW * STAGE <= (EPI == EPI_RES ? C::RES_BYTES : C::REGION_BYTES),
                  "epilogue staging fits in the LDS buffer");
    uint8_t* stage = smem + wave * STAGE;

    // NORM: LayerNorm over the Cout channels of every output position, then the per-channel
    // scale and shift and (optionally) Swish, applied to the float32 sums (bias added) before
    // the single bf16 rounding of the staging below.  A position's channels are spread over
    // the WCH waves of its column block and, within a wave, over the two lane halves; two
    // reductions through LDS (past the staging area) give the mean and then the sum of
    // squared deviations from it.  Every lane sums the WCH partials in the same order, so all
    // channels of a position use the same statistics.
    // per position (frame, column block): nr = 1 / sqrt(variance + eps), nm = -mean * nr
    float nm[EPI == EPI_NORM ? NV : 1][FB], nr[EPI == EPI_NORM ? NV : 1][FB];
    float4 lg[EPI == EPI_NORM ? FA : 1][4], lb[EPI == EPI_NORM ? FA : 1][4];
    if constexpr (EPI == EPI_NORM) {
        constexpr int NC = C::NC, RED = WCH * C::R * NC;  // floats per reduction array
        static_assert(C::NW * STAGE + 2 * RED * 4 <= C::REGION_BYTES, "norm reductions fit in the LDS buffer");
        float* red1 = reinterpret_cast<float*>(smem + C::NW * STAGE);
        float* red2 = red1 + RED;
        const float inv_n = 1.0f / (float)g.Cout;
        bool vq[FA][4];  // Cout % 8 == 0: the 4 channels of a group are all valid or all not
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = (ab0 + a) * 32 + 8 * q + 4 * khalf;
                vq[a][q] = n < g.Cout;
                lg[a][q] = vq[a][q] ? *reinterpret_cast<const float4*>(aux.ln_g + n) : make_float4(0.f, 0.f, 0.f, 0.f);
                lb[a][q] = vq[a][q] ? *reinterpret_cast<const float4*>(aux.ln_b + n) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        // the bias joins the sums once, here
#pragma unroll
        for (int ry = 0; ry < NV; ++ry)
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int cb = 0; cb < FB; ++cb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[ry][a][cb][4 * q + e] += bv[a][q][e];
        auto slot = [&](int w, int ry, int cb) { return (w * C::R + ry) * NC + wpos * 32 * FB + cb * 32 + px; };
        // the sum over the lane's valid channels and its partner lane's: of the values for
        // the mean, of their squared deviations from m for the variance
        auto partial = [&](int ry, int cb, float m, bool squares) {
            float acc_s = 0.0f;
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (vq[a][q]) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = acc[ry][a][cb][4 * q + e];
                            acc_s = squares ? fmaf(v - m, v - m, acc_s) : acc_s + v;
                        }
                    }
            return acc_s + __shfl_xor(acc_s, 32);
        };
#pragma unroll
        for (int ry = 0; ry < NV; ++ry)
#pragma unroll
            for (int cb = 0; cb < FB; ++cb) {
                const float ps = partial(ry, cb, 0.0f, false);
                if (khalf == 0) red1[slot(wch, ry, cb)] = ps;
            }
        __syncthreads();
#pragma unroll
        for (int ry = 0; ry < NV; ++ry)
#pragma unroll
            for (int cb = 0; cb < FB; ++cb) {
                float t = 0.0f;
                for (int w = 0; w < WCH; ++w) t += red1[slot(w, ry, cb)];
                nm[ry][cb] = t * inv_n;
                const float ps = partial(ry, cb, nm[ry][cb], true);
                if (khalf == 0) red2[slot(wch, ry, cb)] = ps;
            }
        __syncthreads();
#pragma unroll
        for (int ry = 0; ry < NV; ++ry)
#pragma unroll
            for (int cb = 0; cb < FB; ++cb) {
                float t = 0.0f;
                for (int w = 0; w < WCH; ++w) t += red2[slot(w, ry, cb)];
                nr[ry][cb] = rsqrtf(t * inv_n + aux.eps);
                nm[ry][cb] *= -nr[ry][cb];  // (v - mean) * rstd = fma(v, rstd, -mean * rstd)
            }
    }
    // the staged value of accumulator element e of group (a, q): the sum with its bias, and for
    // NORM normalised, scaled, shifted and passed through Swish
    auto outv = [&](const f32x16_t& c, int ry, int a, int cb, int q, int e) {
        float v;
        if constexpr (EPI == EPI_NORM) {  // the bias is already in c
            const float4 gq = lg[a][q], bq = lb[a][q];
            const float gv = e == 0 ? gq.x : e == 1 ? gq.y : e == 2 ? gq.z : gq.w;
            const float bw = e == 0 ? bq.x : e == 1 ? bq.y : e == 2 ? bq.z : bq.w;
            v = fmaf(fmaf(c[4 * q + e], nr[ry][cb], nm[ry][cb]), gv, bw);
            if (aux.swish) v = swish_f(v);
        } else {
            v = c[4 * q + e] + bv[a][q][e];
        }
        return v;
    };
    const int nb = (ab0 * 32) * 2;  // byte offset of this wave's first channel in a position row
    constexpr int CPP = 4 * FA;   // 16-byte output chunks per position slice
    constexpr int PPI = 64 / CPP;  // positions per store instruction
    constexpr int NIT = 32 * FB / PPI;
    const int c16 = lane % CPP;
    const int n = ab0 * 32 + c16 * 8;
    // output position of store step it of frame ry, and whether it is stored
    auto out_pos = [&](int ry, int it, long long& pos) {
        const int col = it * PPI + lane / CPP;
        bool ok;
        if (KIND == SPATIAL3) {
            const int y = r0 + ry, x = c0 + wpos * 32 * FB + col;
            ok = x < g.W;
            pos = (((long long)b * g.T + t) * g.H + y) * g.W + x;
        } else {
            const int hw = c0 + wpos * 32 * FB + col;
            ok = hw < g.HW;
            pos = ((long long)b * g.T + r0 + ry) * g.HW + hw;
        }
        return ok && n < g.Cout;  // Cout is a multiple of 8 on this path (checked by the launcher)
    };
    // RES: the residual chunks of every frame of the tile are requested at once, before any
    // staging (unconditional loads, a stored position's chunk or the tensor's first one), so the
    // tile waits for one HBM round trip instead of one per frame; the operand registers of the K
    // loop are free by now.
    uint4 rv[EPI == EPI_RES ? NV : 1][EPI == EPI_RES ? NIT : 1];
    if constexpr (EPI == EPI_RES) {
#pragma unroll
        for (int ry = 0; ry < NV; ++ry)
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                long long pos;
                const bool ok = out_pos(ry, it, pos);
                rv[ry][it] = *reinterpret_cast<const uint4*>(aux.res + (ok ? pos * g.Cout + n : 0));
            }
    }
#pragma unroll
    for (int ry = 0; ry < NV; ++ry) {
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int cb = 0; cb < FB; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16_t& c = acc[ry][a][cb];
                    uint8_t* dst = stage + (cb * 32 + px) * OS + (a * 32 + 8 * q + 4 * khalf) * ES;
                    if constexpr (EPI == EPI_RES) {
                        *reinterpret_cast<float4*>(dst) = make_float4(c[4 * q] + bv[a][q][0], c[4 * q + 1] + bv[a][q][1],
                                                                      c[4 * q + 2] + bv[a][q][2],
                                                                      c[4 * q + 3] + bv[a][q][3]);
                    } else {
                        uint2 u;
                        u.x = pack_bf16x2(outv(c, ry, a, cb, q, 0), outv(c, ry, a, cb, q, 1));
                        u.y = pack_bf16x2(outv(c, ry, a, cb, q, 2), outv(c, ry, a, cb, q, 3));
                        *reinterpret_cast<uint2*>(dst) = u;
                    }
                }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int col = it * PPI + lane / CPP;
            long long pos;
            const bool ok = out_pos(ry, it, pos);
            uint4 v;
            if constexpr (EPI == EPI_RES) {
                const float4 f0 = *reinterpret_cast<const float4*>(stage + col * OS + c16 * 32);
                const float4 f1 = *reinterpret_cast<const float4*>(stage + col * OS + c16 * 32 + 16);
                const uint4 r = rv[ry][it];
                v.x = pack_bf16x2(f0.x + bf16_lo(r.x), f0.y + bf16_hi(r.x));
                v.y = pack_bf16x2(f0.z + bf16_lo(r.y), f0.w + bf16_hi(r.y));
                v.z = pack_bf16x2(f1.x + bf16_lo(r.z), f1.y + bf16_hi(r.z));
                v.w = pack_bf16x2(f1.z + bf16_lo(r.w), f1.w + bf16_hi(r.w));
            } else {
                v = *reinterpret_cast<const uint4*>(stage + col * OS + c16 * 16);
            }
            if (ok) st_stream16(reinterpret_cast<uint8_t*>(Y + pos * g.Cout) + nb + c16 * 16, v);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// rows_tile with a compile-time count of valid output rows
template <typename C, bool TAIL, int EPI, bool HIST>
__device__ __forceinline__ void rows_nv(int nv, const uint16_t* Wf, const uint16_t* X, const float* bias, uint16_t* Y,
                                        const uint16_t* Wpf, const float* bias_p, const uint16_t* Hx,
                                        const RowsGeom& g, const RowsAux& aux, uint8_t* smem, int b, int t, int ct,
                                        int r0, int c0) {
    constexpr int R = C::R;
    if (nv >= R)
        rows_tile<C, R, TAIL, EPI, HIST>(Wf, X, bias, Y, Wpf, bias_p, Hx, g, aux, smem, b, t, ct, r0, c0);
    else if (nv == 3)
        rows_tile<C, (R > 3 ? 3 : R), TAIL, EPI, HIST>(Wf, X, bias, Y, Wpf, bias_p, Hx, g, aux, smem, b, t, ct, r0, c0);
    else if (nv == 2)
        rows_tile<C, (R > 2 ? 2 : R), TAIL, EPI, HIST>(Wf, X, bias, Y, Wpf, bias_p, Hx, g, aux, smem, b, t, ct, r0, c0);
    else
        rows_tile<C, 1, TAIL, EPI, HIST>(Wf, X, bias, Y, Wpf, bias_p, Hx, g, aux, smem, b, t, ct, r0, c0);
}

template <typename C, bool TAIL, int EPI, bool HISTK = false>
__global__ __launch_bounds__(C::NTH) __attribute__((amdgpu_waves_per_eu(2))) void conv_rows_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wf, const float* __restrict__ bias,
    uint16_t* __restrict__ Y, const uint16_t* __restrict__ Wpf, const float* __restrict__ bias_p,
    const uint16_t* __restrict__ Hx, RowsGeom g, RowsAux aux) {
    constexpr int KIND = C::KIND;
    // the region buffers; the fused projection's partial sums reuse them after the K loop
    __shared__ __attribute__((aligned(16))) uint8_t smem[epi_proj<EPI>() ? std::max(C::REGION_BYTES, C::PROJ_BYTES)
                                                                      : EPI == EPI_RES ? std::max(C::REGION_BYTES, C::RES_BYTES)
                                                                                       : C::REGION_BYTES + (C::SRC == SRC_FSQ ? LIFT_BYTES : 0)];

    int tile = (int)(blockIdx.x & 7) * g.per_xcd + (int)(blockIdx.x >> 3);
    if (tile >= g.ntiles) return;
    // tile order (fastest first): channel tile, row tile, column tile, frame, clip; the
    // channel tiles of a region and the row tiles that share its look-back rows run back to
    // back on one XCD
    const int ct = tile % g.nct;
    tile /= g.nct;
    const int rt = tile % g.nrow;
    tile /= g.nrow;
    const int cl = tile % g.ncol;
    tile /= g.ncol;
    int t = 0, b = tile;
    if (KIND == SPATIAL3) {
        t = tile % g.T;
        b = tile / g.T;
    }
    // the rows are split evenly over the nrow = ceil(rows / R) row tiles (13 frames as
    // 4 + 3 + 3 + 3, not 4 + 4 + 4 + 1): a tile's weight traffic does not shrink with its
    // row count, so one short tile costs nearly as much as a full one
    const int rows = KIND == SPATIAL3 ? g.H : g.T;
    const int rbase = rows / g.nrow, rextra = rows - rbase * g.nrow;
    const int nv = rbase + (rt < rextra ? 1 : 0);  // valid output rows (block-uniform, <= R)
    const int r0 = rt * rbase + min(rt, rextra), c0 = cl * C::NC;
    // temporal stream (HISTK): only the tiles whose look-back frames reach before frame 0
    // read the history frames
    if (HISTK && r0 < 2)
        rows_nv<C, TAIL, EPI, HISTK>(nv, Wf, X, bias, Y, Wpf, bias_p, Hx, g, aux, smem, b, t, ct, r0, c0);
    else
        rows_nv<C, TAIL, EPI, false>(nv, Wf, X, bias, Y, Wpf, bias_p, Hx, g, aux, smem, b, t, ct, r0, c0);
}

// Input channel k of the K dimension in the Haar-fused spatial conv (SRC_HAAR): pixel
// channel k / 64, level-1 temporal band q = (k / 32) % 2, m = k % 32 the packet rows rt =
// 2 q + m / 16, rh = (m / 4) % 4, rw = m % 4, which the Haar coefficient channel
// s2 * 24 + s1 * 3 + c holds (s1 the level-1 bands (rt, rh, rw) / 2, s2 the level-2 bands
// (rt, rh, rw) % 2, each as 4 b_t + 2 b_h + b_w).
__host__ __device__ inline int haar_k_channel(int k) {
    const int c = k / 64, q = (k / 32) & 1, m = k & 31;
    const int rt = 2 * q + m / 16, rh = (m / 4) & 3, rw = m & 3;
    const int s1 = ((rt >> 1) << 2) | ((rh >> 1) << 1) | (rw >> 1);
    const int s2 = ((rt & 1) << 2) | ((rh & 1) << 1) | (rw & 1);
    return s2 * 24 + s1 * 3 + c;
}

// Weights in MFMA fragment order for conv_rows_kernel: fragment f = (kc16 * taps + j) * NA
// + ab holds, for lane l, the 8 values w[ab * 32 + l % 32][kc16 * 16 + (l / 32) * 8 + e][j],
// e = 0..7, at element offset (f * 64 + l) * 8 + e; rows past Cout and channels past Cin
// are zero.  Input layout is torch's [Cout][Cin][taps].  haar_k: input channel k is
// haar_k_channel(k) of w (Cin = 192).
__global__ __launch_bounds__(256) void pack_frag_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wf,
                                                        int Cout, int Cin, int ntaps, int NA, int KC16, int haar_k) {
    const long long total = (long long)KC16 * ntaps * NA * 512;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int e = (int)(i & 7), l = (int)((i >> 3) & 63);
        const long long f = i >> 9;
        const int ab = (int)(f % NA);
        const long long f2 = f / NA;
        const int j = (int)(f2 % ntaps), kc16 = (int)(f2 / ntaps);
        const int row = ab * 32 + (l & 31);
        const int k = kc16 * 16 + (l >> 5) * 8 + e;
        const int ks = haar_k ? haar_k_channel(k) : k;
        wf[i] = (row < Cout && k < Cin) ? w[((size_t)row * Cin + ks) * ntaps + j] : (uint16_t)0;
    }
}

size_t frag_bytes(int Cout, int Cin, int ntaps) {
    return (size_t)((Cin + 15) / 16) * ntaps * ((Cout + 31) / 32) * 512 * 2;
}

// Wp[n][tap][c] = w[n][c][tap]  (torch order [Cout][Cin][kernel...] -> K contiguous)
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wp,
                                                           int Cout, int Cin, int ntaps) {
    const long long total = (long long)Cout * Cin * ntaps;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long per = (long long)ntaps * Cin;
        const int n = (int)(i / per);
        const int rem = (int)(i - n * per);
        const int tap = rem / Cin, c = rem - (rem / Cin) * Cin;
        wp[i] = w[((size_t)n * Cin + c) * ntaps + tap];
    }
}

// 1x1 projections with at most 16 input channels (the lift after FSQ dequantize): one item
// per (position, 8 output channels), fp32 FMA in channel order, the bias first.  Items are
// numbered position-major, so consecutive items are consecutive 16-byte chunks of one
// position's output row (coalesced stores).  STAGED (the weights fit SMALL_PROJ_LDS_FLOATS):
// the workgroup converts them once to float32 [c][CS] rows in LDS (CS = Cout rounded up to
// 8, zeros past Cout; row Cin holds the bias), and the grid-stride is a multiple of the ng
// channel groups of a position, so a thread's group never changes: it copies its 8 columns
// of weights into registers once and the loop reads no weights at all.  Otherwise the
// weights are read from global per item.
constexpr int SMALL_PROJ_LDS_FLOATS = 12288;  // 48 KB

__device__ __forceinline__ int small_proj_cs(int Cout) { return (Cout + 7) & ~7; }

template <int CMAX>
struct SmallProjW {
    float w[CMAX][8];
    float b[8];
};

template <int CMAX>
__device__ __forceinline__ void small_proj_regs(const uint16_t* __restrict__ w, const float* __restrict__ bias,
                                                float* sw, int Cin, int Cout, int n0, SmallProjW<CMAX>& r) {
    const int CS = small_proj_cs(Cout);
    for (int i = threadIdx.x; i < (Cin + 1) * CS; i += blockDim.x) {
        const int c = i / CS, n = i - c * CS;
        float v = 0.0f;
        if (n < Cout) v = c < Cin ? bf16_to_f32(w[(size_t)n * Cin + c]) : (bias ? bias[n] : 0.0f);
        sw[i] = v;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) r.w[c][e] = c < Cin ? sw[c * CS + n0 + e] : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.b[e] = sw[Cin * CS + n0 + e];
}

// o[e] = bias[n0 + e] + sum_c w[n0 + e][c] x[c]
template <int CMAX>
__device__ __forceinline__ void small_proj8_regs(const float* xv, int Cin, const SmallProjW<CMAX>& r, float* o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = r.b[e];
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
        if (c < Cin) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(r.w[c][e], xv[c], o[e]);
        }
}

__device__ __forceinline__ void small_proj8_global(const float* xv, int Cin, int Cout, int n0,
                                                   const uint16_t* __restrict__ w, const float* __restrict__ bias,
                                                   float* o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int n = n0 + e;
        float a = 0.0f;
        if (n < Cout) {
            a = bias ? bias[n] : 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (c < Cin) a = fmaf(bf16_to_f32(w[(size_t)n * Cin + c]), xv[c], a);
        }
        o[e] = a;
    }
}

__device__ __forceinline__ void small_proj_store(uint16_t* __restrict__ Y, long long pos, int Cout, int n0,
                                                 const float* o) {
    uint16_t* yrow = Y + (size_t)pos * Cout;
    if ((Cout & 7) == 0) {
        uint4 u;
        u.x = pack_bf16x2(o[0], o[1]);
        u.y = pack_bf16x2(o[2], o[3]);
        u.z = pack_bf16x2(o[4], o[5]);
        u.w = pack_bf16x2(o[6], o[7]);
        st_stream16(yrow + n0, u);  // written once, read back only by the next kernel
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (n0 + e < Cout) yrow[n0 + e] = f32_to_bf16(o[e]);
    }
}

// CMAX = 0: weights from global; else staged, CMAX >= Cin
template <int CMAX>
__global__ __launch_bounds__(256) void pointwise_small_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ w,
                                                              const float* __restrict__ bias, uint16_t* __restrict__ Y,
                                                              long long P, int Cin, int Cout) {
    extern __shared__ __attribute__((aligned(16))) float sw[];
    const int ng = (Cout + 7) / 8;
    const long long total = P * ng;
    const long long first = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int n0 = (int)(first % ng) * 8;  // fixed: the stride is a multiple of ng
    SmallProjW<(CMAX > 0 ? CMAX : 1)> r;
    if constexpr (CMAX > 0) small_proj_regs<CMAX>(w, bias, sw, Cin, Cout, n0, r);
    // the position advances by a constant (no 64-bit division per item)
    const long long stride = (long long)gridDim.x * blockDim.x, dpos = stride / ng;
    long long pos = first / ng;
    for (long long item = first; item < total; item += stride, pos += dpos) {
        float xv[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) xv[c] = c < Cin ? bf16_to_f32(X[(size_t)pos * Cin + c]) : 0.0f;
        float o[8];
        if constexpr (CMAX > 0)
            small_proj8_regs<CMAX>(xv, Cin, r, o);
        else
            small_proj8_global(xv, Cin, Cout, n0, w, bias, o);
        small_proj_store(Y, pos, Cout, n0, o);
    }
}

// FSQ dequantize fused with the 1x1 projection D -> Cout that follows it in the decoder.
// The index is split into digits by exact multiply-shift divisions, each code
// (d - L/2) / (L/2) is rounded to bf16 (what the dequantize kernel stores) and the
// projection accumulates exactly as pointwise_small_kernel does, so the result is
// bit-identical to the two kernels in a row while the D-channel codes never reach HBM.  An
// index outside [0, codebook) gives NaN outputs and is counted once per position in
// *invalid (one atomic per wave and step; the loop's trip count is uniform per wave).
// DEF: the default level set (8, 8, 8, 5, 5, 5), whose digits are the three 3-bit fields of
// idx mod 512 and the base-5 digits of q = idx / 512 < 125, split by q / 5 = (q * 205) >> 10
// (exact for q < 1024): about 10 operations per index instead of six general divisions, the
// same digits and codes.
template <int CMAX, bool DEF = false>
__global__ __launch_bounds__(256) void fsq_dequant_proj_kernel(const int32_t* __restrict__ idx, FsqParams p,
                                                               const uint16_t* __restrict__ w,
                                                               const float* __restrict__ bias,
                                                               uint16_t* __restrict__ Y, long long P, int Cout,
                                                               int32_t* __restrict__ invalid) {
    extern __shared__ __attribute__((aligned(16))) float sw[];
    const int ng = (Cout + 7) / 8;
    const long long total = P * ng;
    const int lane = threadIdx.x & 63;
    const long long first = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int n0 = (int)(first % ng) * 8;  // fixed: the stride is a multiple of ng
    SmallProjW<(CMAX > 0 ? CMAX : 1)> r;
    if constexpr (CMAX > 0) small_proj_regs<CMAX>(w, bias, sw, p.D, Cout, n0, r);
    // the position advances by a constant (no 64-bit division per item); U items per step,
    // their index loads issued together
    constexpr int U = 4;
    const long long stride = (long long)gridDim.x * blockDim.x, dpos = stride / ng;
    long long pos = first / ng;
    for (long long base = first - lane; base < total; base += U * stride, pos += U * dpos) {
        int ids[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ids[u] = base + u * stride + lane < total ? idx[pos + u * dpos] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
        const long long item = base + u * stride + lane;
        const bool live = item < total;
        const int id = ids[u];
        const bool bad = id < 0 || id >= p.codebook;
        if (invalid) {
            const unsigned long long m = __builtin_amdgcn_ballot_w64(live && bad && n0 == 0);
            if (m && lane == (int)__builtin_ctzll(m)) atomicAdd(invalid, (int)__builtin_popcountll(m));
        }
        if (!live) continue;
        uint32_t rem = bad ? 0u : (uint32_t)id;
        float xv[16];
        if constexpr (DEF) {
            const uint32_t q = rem >> 9, q5 = (q * 205u) >> 10, q25 = (q5 * 205u) >> 10;
            const int d[6] = {(int)(rem & 7u), (int)((rem >> 3) & 7u), (int)((rem >> 6) & 7u), (int)(q - 5u * q5),
                              (int)(q5 - 5u * q25), (int)q25};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float code = i < 3 ? (float)(d[i] - 4) * 0.25f : (float)(d[i < 6 ? i : 5] - 2) * 0.5f;
                xv[i] = i < 6 ? (bad ? __builtin_nanf("") : bf16_to_f32(f32_to_bf16(code))) : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (DEF) break;
            xv[i] = 0.0f;
            if (i < FSQ_MAX_D && i < p.D) {
                const uint32_t q = div_magic(rem, p.magic[i], p.shift[i]);
                const int d = (int)(rem - q * (uint32_t)p.levels[i]);
                rem = q;
                // (d - h) / h; for a power-of-two h (every level of the default set) the product
                // with the exact reciprocal is the same float, without a division
                const int h = p.half[i];
                const float code = (h & (h - 1)) == 0 ? (float)(d - h) * (1.0f / (float)h) : (float)(d - h) / (float)h;
                xv[i] = bad ? __builtin_nanf("") : bf16_to_f32(f32_to_bf16(code));
            }
        }
        float o[8];
        if constexpr (CMAX > 0)
            small_proj8_regs<CMAX>(xv, p.D, r, o);
        else
            small_proj8_global(xv, p.D, Cout, n0, w, bias, o);
        small_proj_store(Y, pos + u * dpos, Cout, n0, o);
        }
    }
}

// Grid of the small projections: at most about 4096 workgroups, rounded up to a multiple of
// ng / gcd(ng, 256) so that the grid-stride is a multiple of the ng channel groups.
inline long long small_proj_blocks(long long items, int ng) {
    long long a = ng, b = 256;
    while (b) {
        const long long t = a % b;
        a = b;
        b = t;
    }
    const long long m = ng / a;
    const long long nb = std::min((items + 255) / 256, 4096LL);
    return (nb + m - 1) / m * m;
}
inline size_t small_proj_lds(int Cin, int Cout) { return (size_t)(Cin + 1) * ((Cout + 7) & ~7) * sizeof(float); }
inline bool small_proj_staged(int Cin, int Cout) {
    return (long long)(Cin + 1) * ((Cout + 7) & ~7) <= SMALL_PROJ_LDS_FLOATS;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

template <int KIND, int TC, int TP, int WC, int WP>
hipError_t launch_igemm_t(const uint16_t* X, const uint16_t* Wp, const float* bias, uint16_t* Y, const ConvGeom& g,
                          hipStream_t s) {
    const long long ntp = (g.P + TP - 1) / TP;
    const long long ntc = (g.Cout + TC - 1) / TC;
    const long long nblk = ntp * ntc;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((conv_igemm_kernel<KIND, TC, TP, WC, WP>), dim3((unsigned)nblk), dim3(256), 0, s, X, Wp, bias,
                       Y, g);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_igemm_k(const uint16_t* X, const uint16_t* Wp, const float* bias, uint16_t* Y, const ConvGeom& g,
                          hipStream_t s) {
    if (g.Cout <= 32) return launch_igemm_t<KIND, 32, 128, 1, 4>(X, Wp, bias, Y, g, s);
    if (g.Cout <= 64) return launch_igemm_t<KIND, 64, 128, 1, 4>(X, Wp, bias, Y, g, s);
    if (g.Cout <= 128) return launch_igemm_t<KIND, 128, 128, 2, 2>(X, Wp, bias, Y, g, s);
    if (g.Cout <= 192) return launch_igemm_t<KIND, 192, 128, 2, 2>(X, Wp, bias, Y, g, s);
    return launch_igemm_t<KIND, 256, 128, 2, 2>(X, Wp, bias, Y, g, s);
}

// Tile configurations of conv_rows_kernel (see RowsCfg).  Spatial: 4 channel waves of 32
// channels x 64 pixels (128 x 64 per workgroup, three weight fragments per step per wave)
// up to 128 output channels, else 4 waves of 64 x 32 (256 x 32 per workgroup, six
// fragments per step requested early), 2% faster on the 720p layers.  Temporal: 4 waves of
// 32 x 64 up to 128 channels; 4 waves of 64 channels x 32 positions up to 256 (two
// workgroups per CU, so their waves are not all tied by one barrier and one's epilogue
// overlaps the other's MFMAs: 3-10% faster than 8 waves of 32 x 64 in one workgroup, which
// remain above 256 channels).
#ifndef CVT_ROWS_SP_WCH
#define CVT_ROWS_SP_WCH 4
#endif
#ifndef CVT_ROWS_SP_FA
#define CVT_ROWS_SP_FA 1
#endif
#ifndef CVT_ROWS_SP_NW
#define CVT_ROWS_SP_NW 4
#endif
#ifndef CVT_ROWS_SP_BK
#define CVT_ROWS_SP_BK 32
#endif
using SpatialCfg = RowsCfg<SPATIAL3, 4, CVT_ROWS_SP_WCH, CVT_ROWS_SP_FA, CVT_ROWS_SP_BK, CVT_ROWS_SP_NW>;
// 256 channels x 32 columns (two 32-channel blocks per wave, weight fragments requested early):
// the default; 2% faster than 128 x 64 on the 720p layers, and it pads less on some shapes (192
// channels on 160-column rows: 1.33x the work instead of 1.6x)
using SpatialWideCfg = RowsCfg<SPATIAL3, 4, 4, 2, 32, 4>;
// the same tiles staging computed regions (cross-stage fusion): Haar of pixels, dequantized FSQ
using SpatialHaarCfg = RowsCfg<SPATIAL3, 4, 4, 2, 32, 4, 1, SRC_HAAR>;
using SpatialFsqCfg = RowsCfg<SPATIAL3, 4, 4, 2, 32, 4, 1, SRC_FSQ>;
#ifndef CVT_ROWS_TM_BK
#define CVT_ROWS_TM_BK 32
#endif
using TemporalCfg = RowsCfg<TEMPORAL3, 4, 8, 1, CVT_ROWS_TM_BK, 8>;
using TemporalNarrowCfg = RowsCfg<TEMPORAL3, 4, 4, 1, CVT_ROWS_TM_BK, 4>;
using TemporalProjCfg = RowsCfg<TEMPORAL3, 4, 4, 2, CVT_ROWS_TM_BK, 4>;
// 129..192 output channels without padding them to 256: 3 waves of 64 channels x 32 columns
// (two 3-wave workgroups per CU, 6 of the 8 wave slots; on 192 -> 192 at 8 x 13 x 90 x 160
// the spatial conv runs 12% and the temporal conv 8% faster than on the padded 4-wave
// tiles).  The computed-region variant holds 3 rows (5 x 34 region rows for 192 threads).
using SpatialTriCfg = RowsCfg<SPATIAL3, 4, 3, 2, 32, 3>;
using SpatialFsqTriCfg = RowsCfg<SPATIAL3, 3, 3, 2, 32, 3, 1, SRC_FSQ>;
using TemporalTriCfg = RowsCfg<TEMPORAL3, 4, 3, 2, CVT_ROWS_TM_BK, 3>;

// conv_rows_kernel over an NTHWC input: Cout % 8 == 0, a tile's input span below ROWS_OOB_BASE
// bytes (use_rows_kernel).
// With Wpf (temporal only, Cout <= 256, Cp <= 16) the epilogue applies the 1x1 projection
// to Cp channels and Y is the [positions][Cp] projected output.
template <typename C, bool TAIL, int EPI>
hipError_t launch_rows_k(const uint16_t* X, const uint16_t* Wf, const float* bias, uint16_t* Y, const uint16_t* Wpf,
                         const float* bias_p, const uint16_t* Hx, const RowsGeom& g, const RowsAux& aux,
                         hipStream_t s) {
    const dim3 grid((unsigned)(8LL * g.per_xcd)), block(C::NTH);
    if constexpr (C::KIND == TEMPORAL3 && C::S == 1 && (EPI == EPI_PLAIN || EPI == EPI_PROJ)) {
        if (Hx) {
            hipLaunchKernelGGL((conv_rows_kernel<C, TAIL, EPI, true>), grid, block, 0, s, X, Wf, bias, Y, Wpf, bias_p,
                               Hx, g, aux);
            return hipGetLastError();
        }
    }
    if (Hx) return hipErrorInvalidValue;
    hipLaunchKernelGGL((conv_rows_kernel<C, TAIL, EPI, false>), grid, block, 0, s, X, Wf, bias, Y, Wpf, bias_p, Hx, g,
                       aux);
    return hipGetLastError();
}

template <typename C, int EPI>
hipError_t launch_rows_tail(bool tail, const uint16_t* X, const uint16_t* Wf, const float* bias, uint16_t* Y,
                            const uint16_t* Wpf, const float* bias_p, const uint16_t* Hx, const RowsGeom& g,
                            const RowsAux& aux, hipStream_t s) {
    return tail ? launch_rows_k<C, true, EPI>(X, Wf, bias, Y, Wpf, bias_p, Hx, g, aux, s)
                : launch_rows_k<C, false, EPI>(X, Wf, bias, Y, Wpf, bias_p, Hx, g, aux, s);
}

// Hx (temporal only): the two frames before X, [B][2][HW][Cin] NTHWC, read in place of the
// causal zero padding (a chunk of a stream); nullptr = zero padding.  aux selects the NORM
// (aux.ln_g set) or RES (aux.res set) epilogue.
template <typename C>
hipError_t launch_rows_cfg(const uint16_t* X, const uint16_t* Wf, const float* bias, uint16_t* Y, const ConvGeom& cg,
                           int B, hipStream_t s, const uint16_t* Wpf, const float* bias_p, int Cp,
                           const uint16_t* Hx, const RowsAux& aux) {
    constexpr int KIND = C::KIND, R = C::R, BK = C::BK;
    RowsGeom g{};
    g.B = B; g.T = cg.T; g.H = cg.H; g.W = cg.W; g.HW = cg.H * cg.W; g.Cin = cg.Cin; g.Cout = cg.Cout;
    g.ups = cg.ups;
    const bool in_grid = cg.ups || C::S == 2;  // the input grid differs from the output grid
    g.Ti = in_grid ? cg.Ti : cg.T;
    g.Hi = in_grid ? cg.Hi : cg.H;
    g.Wi = in_grid ? cg.Wi : cg.W;
    if (C::S == 2 && cg.ups) return hipErrorInvalidValue;
    g.x_total = (long long)B * g.Ti * g.Hi * g.Wi * cg.Cin * 2;
    if constexpr (C::SRC == SRC_HAAR) g.x_total = (long long)B * 3 * aux.px_T * 16 * cg.H * cg.W * 2;
    if constexpr (C::SRC == SRC_FSQ) g.x_total = (long long)B * cg.T * cg.H * cg.W * 4;
    if (cg.ups && Hx) return hipErrorInvalidValue;
    g.wf_bytes = (int)frag_bytes(cg.Cout, cg.Cin, KIND == SPATIAL3 ? 9 : 3);
    g.NA = (cg.Cout + 31) / 32;
    g.KC16 = (cg.Cin + 15) / 16;
    g.nct = (cg.Cout + C::TCH - 1) / C::TCH;
    g.Cp = Cp;
    g.wp_bytes = Wpf ? (int)frag_bytes(Cp, cg.Cout, 1) : 0;
    g.h_total = Hx ? (long long)B * 2 * g.HW * cg.Cin * 2 : 0;
    long long ntiles;
    if (KIND == SPATIAL3) {
        g.ncol = (cg.W + C::NC - 1) / C::NC;
        g.nrow = (cg.H + R - 1) / R;
        ntiles = (long long)g.nct * g.ncol * g.nrow * cg.T * B;
    } else {
        g.ncol = (g.HW + C::NC - 1) / C::NC;
        g.nrow = (cg.T + R - 1) / R;
        ntiles = (long long)g.nct * g.ncol * g.nrow * B;
    }
    if (ntiles > 0x7ffffff0LL) return hipErrorInvalidConfiguration;
    g.ntiles = (int)ntiles;
    g.per_xcd = (int)((ntiles + 7) / 8);
    const bool tail = cg.Cin % BK != 0;
    if constexpr (KIND == TEMPORAL3 && (C::NW == 4 || C::NW == 3) && C::S == 1) {  // 3- and 4-wave temporal tiles: projection, norm
        if (Wpf) {
            if (g.nct != 1 || Cp < 1 || Cp > 16 || aux.ln_g || aux.res) return hipErrorInvalidValue;
            if (aux.fsq_idx) {
                if (Cp != aux.fsq.D || Cp > 8 || Hx) return hipErrorInvalidValue;
                return launch_rows_tail<C, EPI_PFSQ>(tail, X, Wf, bias, Y, Wpf, bias_p, Hx, g, aux, s);
            }
            return launch_rows_tail<C, EPI_PROJ>(tail, X, Wf, bias, Y, Wpf, bias_p, Hx, g, aux, s);
        }
        if (aux.ln_g) {
            if (g.nct != 1 || aux.res) return hipErrorInvalidValue;
            return launch_rows_tail<C, EPI_NORM>(tail, X, Wf, bias, Y, nullptr, nullptr, Hx, g, aux, s);
        }
    }
    if (Wpf || aux.ln_g) return hipErrorInvalidValue;
    if constexpr (KIND == TEMPORAL3 && C::S == 1) {  // residual epilogue (4-wave tiles up to 256 channels, else 8-wave)
        if (aux.res) return launch_rows_tail<C, EPI_RES>(tail, X, Wf, bias, Y, nullptr, nullptr, Hx, g, aux, s);
    }
    if (aux.res) return hipErrorInvalidValue;
    return launch_rows_tail<C, EPI_PLAIN>(tail, X, Wf, bias, Y, nullptr, nullptr, Hx, g, aux, s);
}

template <int KIND>
hipError_t launch_rows(const uint16_t* X, const uint16_t* Wf, const float* bias, uint16_t* Y, const ConvGeom& cg,
                       int B, hipStream_t s, const uint16_t* Wpf = nullptr, const float* bias_p = nullptr,
                       int Cp = 0, const uint16_t* Hx = nullptr, const RowsAux& aux = RowsAux{}) {
    if constexpr (KIND == SPATIAL3) {
        // the tile shape that pads the output channels and row columns least (ties: 256 x 32;
        // 128 x 64 wins for up to 128 output channels)
        auto padded = [&](int tch, int nc) {
            return (long long)((cg.Cout + tch - 1) / tch) * tch * (long long)(((cg.W + nc - 1) / nc) * nc);
        };
        if (cg.Cout > 128 && cg.Cout <= SpatialTriCfg::TCH)
            return launch_rows_cfg<SpatialTriCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, nullptr, aux);
        if (padded(SpatialCfg::TCH, SpatialCfg::NC) < padded(SpatialWideCfg::TCH, SpatialWideCfg::NC))
            return launch_rows_cfg<SpatialCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, nullptr, aux);
        return launch_rows_cfg<SpatialWideCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, nullptr, aux);
    }
    if (cg.Cout <= TemporalNarrowCfg::TCH)
        return launch_rows_cfg<TemporalNarrowCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, Hx, aux);
    // up to 256 channels: 4-wave tiles of two 32-channel blocks per wave, two workgroups per CU, so
    // one's epilogue (projection, norm, residual or plain stores) overlaps the other's MFMAs, with
    // the weight fragments requested right after their last use (also 2.5-10% faster than the
    // 8-wave tiles for the plain conv)
    if (cg.Cout <= TemporalTriCfg::TCH)
        return launch_rows_cfg<TemporalTriCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, Hx, aux);
    if (cg.Cout <= TemporalProjCfg::TCH)
        return launch_rows_cfg<TemporalProjCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, Hx, aux);
    return launch_rows_cfg<TemporalCfg>(X, Wf, bias, Y, cg, B, s, Wpf, bias_p, Cp, Hx, aux);
}

// The stride-2 (downsampling) convolutions on conv_rows_kernel: cg holds the output grid
// and, in Ti, Hi, Wi, the input grid.  Spatial tiles of 256 channels x 32 columns x 3 output
// rows (7 input rows of 65 de-interleaved columns, each region staged once for 256 output
// channels; the two 80 KB region buffers still let two workgroups share a CU, and a weight
// fragment feeds 3 MFMAs: 14% faster than 2 output rows, 1.46x faster than 128 x 64 tiles on
// 256 -> 256), or 128 x 64 x 1 up to 128 channels (3 input rows of 129 columns, two
// workgroups per CU); temporal tiles as at stride 1 with 9 input frames per 4 output frames
// (5 per 2 on the 8-wave tiles above 256 channels).
using SpatialS2NarrowCfg = RowsCfg<SPATIAL3, 1, 4, 1, 32, 4, 2>;
using SpatialS2Cfg = RowsCfg<SPATIAL3, 3, 4, 2, 32, 4, 2>;
using TemporalS2NarrowCfg = RowsCfg<TEMPORAL3, 3, 4, 1, 32, 4, 2>;  // 7 staged frames x 64 columns: 72 KB
using TemporalS2Cfg = RowsCfg<TEMPORAL3, 4, 4, 2, 32, 4, 2>;
using TemporalS2WideCfg = RowsCfg<TEMPORAL3, 2, 8, 1, 32, 8, 2>;  // 2 output frames: 5 staged rows fit the registers

template <int KIND>
hipError_t launch_rows_s2(const uint16_t* X, const uint16_t* Wf, const float* bias, uint16_t* Y, const ConvGeom& cg,
                          int B, hipStream_t s) {
    const RowsAux none{};
    if constexpr (KIND == SPATIAL3) {
        if (cg.Cout <= SpatialS2NarrowCfg::TCH)
            return launch_rows_cfg<SpatialS2NarrowCfg>(X, Wf, bias, Y, cg, B, s, nullptr, nullptr, 0, nullptr, none);
        return launch_rows_cfg<SpatialS2Cfg>(X, Wf, bias, Y, cg, B, s, nullptr, nullptr, 0, nullptr, none);
    }
    if (cg.Cout <= TemporalS2NarrowCfg::TCH)
        return launch_rows_cfg<TemporalS2NarrowCfg>(X, Wf, bias, Y, cg, B, s, nullptr, nullptr, 0, nullptr, none);
    if (cg.Cout <= TemporalS2Cfg::TCH)
        return launch_rows_cfg<TemporalS2Cfg>(X, Wf, bias, Y, cg, B, s, nullptr, nullptr, 0, nullptr, none);
    return launch_rows_cfg<TemporalS2WideCfg>(X, Wf, bias, Y, cg, B, s, nullptr, nullptr, 0, nullptr, none);
}

// Largest Cout whose temporal conv can take the NORM epilogue (all channels in one workgroup).
constexpr int ROWS_NORM_MAX_C = TemporalProjCfg::TCH;

hipError_t launch_igemm(int kind, const uint16_t* X, const uint16_t* Wp, const float* bias, uint16_t* Y,
                        const ConvGeom& g0, hipStream_t s) {
    ConvGeom g = g0;
    if (g.st == 0) {  // stride 1 on the output grid
        g.Ti = g.T; g.Hi = g.H; g.Wi = g.W; g.st = 1; g.ss = 1;
    }
    if (g.ups) return hipErrorInvalidValue;
    if (kind == SPATIAL3) return launch_igemm_k<SPATIAL3>(X, Wp, bias, Y, g, s);
    if (kind == TEMPORAL3) return launch_igemm_k<TEMPORAL3>(X, Wp, bias, Y, g, s);
    return launch_igemm_k<POINT>(X, Wp, bias, Y, g, s);
}

hipError_t pack(const void* w, uint16_t* wp, int Cout, int Cin, int ntaps, hipStream_t s) {
    const long long total = (long long)Cout * Cin * ntaps;
    long long nblk = (total + 255) / 256;
    if (nblk > 65535) nblk = 65535;
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)nblk), dim3(256), 0, s, (const uint16_t*)w, wp, Cout, Cin,
                       ntaps);
    return hipGetLastError();
}

}  // namespace

// packed weights of one convolution: the larger of the fragment order used by
// conv_rows_kernel and the [Cout][tap][Cin] order used by the other kernels
size_t pack_bytes(int Cout, int Cin, int ntaps) {
    return align256(std::max((size_t)Cout * Cin * ntaps * 2, frag_bytes(Cout, Cin, ntaps)));
}

// conv_rows_kernel takes a k = 3 conv with Cout >= 64, Cout % 8 == 0 when a tile's region fits
// its 31-bit buffer offsets: span = input positions between a tile's first and last staged
// row (spatial: 10 image rows of the input; temporal: 9 frames of the input, the stride-2 tiles'
// reach), whatever the tensor's total size.
long long rows_span_spatial(int W_in) { return 10LL * W_in; }
long long rows_span_temporal(long long HW_in) { return 9LL * HW_in; }
bool use_rows_kernel(int k, int Cout, long long span, int Cin) {
    return k == 3 && Cout >= 64 && Cout % 8 == 0 && span * Cin * 2 + 65536 < ROWS_OOB_BASE;
}

hipError_t pack_frag(const void* w, uint16_t* wf, int Cout, int Cin, int ntaps, hipStream_t s, int haar_k = 0) {
    const int NA = (Cout + 31) / 32, KC16 = (Cin + 15) / 16;
    const long long total = (long long)KC16 * ntaps * NA * 512;
    const long long nblk = std::min((total + 255) / 256, 65535LL);
    hipLaunchKernelGGL(pack_frag_kernel, dim3((unsigned)nblk), dim3(256), 0, s, (const uint16_t*)w, wf, Cout, Cin,
                       ntaps, NA, KC16, haar_k);
    return hipGetLastError();
}

size_t conv_workspace_bytes(int B, int Cin, int Cout, int T, int H, int W, int k, bool spatial, bool temporal) {
    const size_t P = (size_t)B * T * H * W;
    size_t b = 0;
    if (spatial) b += pack_bytes(Cout, Cin, k * k);
    if (temporal) b += pack_bytes(Cout, Cout, k);
    if (spatial && temporal) b += align256(P * Cout * 2);
    return b;
}

hipError_t launch_conv_fact(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                            void* y, int B, int Cin, int Cout, int T, int H, int W, int k, void* workspace,
                            hipStream_t s) {
    const long long P = (long long)B * T * H * W;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    size_t off = 0;
    uint16_t* wps = nullptr;
    uint16_t* wpt = nullptr;
    uint16_t* S = nullptr;
    if (w_s) {
        wps = reinterpret_cast<uint16_t*>(ws + off);
        off += pack_bytes(Cout, Cin, k * k);
    }
    if (w_t) {
        wpt = reinterpret_cast<uint16_t*>(ws + off);
        off += pack_bytes(Cout, Cout, k);
    }
    if (w_s && w_t) S = reinterpret_cast<uint16_t*>(ws + off);
    hipError_t e;

    // spatial part: Cin -> Cout, into S (or y when there is no temporal part)
    const uint16_t* tin = static_cast<const uint16_t*>(x);
    if (w_s) {
        uint16_t* sout = w_t ? S : static_cast<uint16_t*>(y);
        if (Cin % 8 != 0) {
            // small-Cin 1x1 path (k == 1 is enforced by the ABI): weights used as [Cout][Cin]
            const int ng = (Cout + 7) / 8;
            const dim3 grid((unsigned)small_proj_blocks(P * ng, ng));
            if (small_proj_staged(Cin, Cout) && Cin <= 8)
                hipLaunchKernelGGL(pointwise_small_kernel<8>, grid, dim3(256), small_proj_lds(Cin, Cout), s,
                                   (const uint16_t*)x, (const uint16_t*)w_s, b_s, sout, P, Cin, Cout);
            else if (small_proj_staged(Cin, Cout))
                hipLaunchKernelGGL(pointwise_small_kernel<16>, grid, dim3(256), small_proj_lds(Cin, Cout), s,
                                   (const uint16_t*)x, (const uint16_t*)w_s, b_s, sout, P, Cin, Cout);
            else
                hipLaunchKernelGGL(pointwise_small_kernel<0>, grid, dim3(256), 0, s, (const uint16_t*)x,
                                   (const uint16_t*)w_s, b_s, sout, P, Cin, Cout);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        } else {
            ConvGeom g{};
            g.P = P; g.T = T; g.H = H; g.W = W; g.Cin = Cin; g.Cout = Cout;
            g.kchunks = (Cin + BK - 1) / BK;
            if (use_rows_kernel(k, Cout, rows_span_spatial(W), Cin)) {
                if ((e = pack_frag(w_s, wps, Cout, Cin, 9, s)) != hipSuccess) return e;
                if ((e = launch_rows<SPATIAL3>((const uint16_t*)x, wps, b_s, sout, g, B, s)) != hipSuccess) return e;
            } else {
                if ((e = pack(w_s, wps, Cout, Cin, k * k, s)) != hipSuccess) return e;
                if ((e = launch_igemm(k == 3 ? SPATIAL3 : POINT, (const uint16_t*)x, wps, b_s, sout, g, s)) !=
                    hipSuccess)
                    return e;
            }
        }
        tin = S;
    }
    if (!w_t) return hipSuccess;

    // temporal part: Cout -> Cout (its input is x itself when there is no spatial part)
    ConvGeom g{};
    g.P = P; g.T = T; g.H = H; g.W = W; g.Cin = Cout; g.Cout = Cout;
    g.kchunks = (Cout + BK - 1) / BK;
    if (use_rows_kernel(k, Cout, rows_span_temporal((long long)H * W), Cout)) {
        if ((e = pack_frag(w_t, wpt, Cout, Cout, 3, s)) != hipSuccess) return e;
        return launch_rows<TEMPORAL3>(tin, wpt, b_t, static_cast<uint16_t*>(y), g, B, s);
    }
    if ((e = pack(w_t, wpt, Cout, Cout, k, s)) != hipSuccess) return e;
    return launch_igemm(k == 3 ? TEMPORAL3 : POINT, tin, wpt, b_t, static_cast<uint16_t*>(y), g, s);
}

// The factorized conv of the Haar coefficients of a 3-channel bf16 clip [B, 3, T, H, W]
// (T = 1 + 4k, causal first frame), the coefficients computed while the spatial conv stages
// its input (SpatialHaarCfg) and never written.  Workspace: the packed spatial weights (in
// the staged channel order) and, with the temporal part, its packed weights and the bf16
// spatial output.
size_t haar_conv_workspace_bytes(int B, int Cout, int T, int H, int W, bool temporal) {
    const size_t P = (size_t)B * (1 + (T - 1) / 4) * (H / 4) * (W / 4);
    size_t b = pack_bytes(Cout, 192, 9);
    if (temporal) b += pack_bytes(Cout, Cout, 3) + align256(P * Cout * 2);
    return b;
}

hipError_t launch_haar_conv(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                            void* y, int B, int Cout, int T, int H, int W, void* workspace, hipStream_t s) {
    const int Tq = 1 + (T - 1) / 4, Hq = H / 4, Wq = W / 4;
    const long long P = (long long)B * Tq * Hq * Wq;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* wps = reinterpret_cast<uint16_t*>(ws);
    size_t off = pack_bytes(Cout, 192, 9);
    uint8_t* tws = ws + off;
    uint16_t* S = w_t ? reinterpret_cast<uint16_t*>(tws + pack_bytes(Cout, Cout, 3)) : static_cast<uint16_t*>(y);
    hipError_t e;
    if ((e = pack_frag(w_s, wps, Cout, 192, 9, s, 1)) != hipSuccess) return e;
    ConvGeom g{};
    g.P = P; g.T = Tq; g.H = Hq; g.W = Wq; g.Cin = 192; g.Cout = Cout;
    g.kchunks = 192 / BK;
    RowsAux aux{};
    aux.px_T = T;
    if ((e = launch_rows_cfg<SpatialHaarCfg>(static_cast<const uint16_t*>(x), wps, b_s, S, g, B, s, nullptr, nullptr,
                                             0, nullptr, aux)) != hipSuccess)
        return e;
    if (!w_t) return hipSuccess;
    return launch_conv_fact(S, nullptr, w_t, nullptr, b_t, y, B, Cout, Cout, Tq, Hq, Wq, 3, tws, s);
}

// The factorized conv of the D -> Cmid projection of dequantized FSQ indices [B, T, H, W],
// the projection computed while the spatial conv stages its input (SpatialFsqCfg).
size_t fsq_conv_workspace_bytes(int B, int Cmid, int Cout, int T, int H, int W, bool temporal) {
    const size_t P = (size_t)B * T * H * W;
    size_t b = pack_bytes(Cout, Cmid, 9);
    if (temporal) b += pack_bytes(Cout, Cout, 3) + align256(P * Cout * 2);
    return b;
}

hipError_t launch_fsq_conv(const int32_t* idx, const FsqParams& p, const void* w_lift, const float* b_lift,
                           const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y, int B,
                           int Cmid, int Cout, int T, int H, int W, void* workspace, hipStream_t s) {
    const long long P = (long long)B * T * H * W;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* wps = reinterpret_cast<uint16_t*>(ws);
    uint8_t* tws = ws + pack_bytes(Cout, Cmid, 9);
    uint16_t* S = w_t ? reinterpret_cast<uint16_t*>(tws + pack_bytes(Cout, Cout, 3)) : static_cast<uint16_t*>(y);
    hipError_t e;
    if ((e = pack_frag(w_s, wps, Cout, Cmid, 9, s)) != hipSuccess) return e;
    ConvGeom g{};
    g.P = P; g.T = T; g.H = H; g.W = W; g.Cin = Cmid; g.Cout = Cout;
    g.kchunks = Cmid / BK;
    RowsAux aux{};
    aux.fsq = p;
    aux.lift_w = static_cast<const uint16_t*>(w_lift);
    aux.lift_b = b_lift;
    e = Cout > 128 && Cout <= SpatialFsqTriCfg::TCH
            ? launch_rows_cfg<SpatialFsqTriCfg>(reinterpret_cast<const uint16_t*>(idx), wps, b_s, S, g, B, s, nullptr,
                                                nullptr, 0, nullptr, aux)
            : launch_rows_cfg<SpatialFsqCfg>(reinterpret_cast<const uint16_t*>(idx), wps, b_s, S, g, B, s, nullptr,
                                             nullptr, 0, nullptr, aux);
    if (e != hipSuccess) return e;
    if (!w_t) return hipSuccess;
    return launch_conv_fact(S, nullptr, w_t, nullptr, b_t, y, B, Cout, Cout, T, H, W, 3, tws, s);
}

namespace {
// the fused projection applies when the temporal part runs on conv_rows_kernel with every
// output channel in one workgroup
bool proj_fused(int k, int Cout, int Cp, long long HW, bool temporal) {
    return temporal && use_rows_kernel(k, Cout, rows_span_temporal(HW), Cout) && Cout <= 256 && Cp <= 16;
}
}  // namespace

size_t conv_proj_workspace_bytes(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k, bool spatial,
                                 bool temporal) {
    const long long P = (long long)B * T * H * W;
    if (proj_fused(k, Cout, Cp, (long long)H * W, temporal)) {
        size_t b = pack_bytes(Cout, Cout, k) + align256(frag_bytes(Cp, Cout, 1));
        if (spatial) b += pack_bytes(Cout, Cin, k * k) + align256((size_t)P * Cout * 2);
        return b;
    }
    return conv_workspace_bytes(B, Cin, Cout, T, H, W, k, spatial, temporal) + align256((size_t)P * Cout * 2) +
           conv_workspace_bytes(B, Cout, Cp, T, H, W, 1, true, false);
}

size_t conv_proj_fsq_workspace_bytes(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k, bool spatial,
                                     bool temporal) {
    return conv_proj_workspace_bytes(B, Cin, Cout, Cp, T, H, W, k, spatial, temporal) +
           align256((size_t)B * T * H * W * Cp * 2);
}

hipError_t launch_conv_fact_proj(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                                 const void* w_p, const float* b_p, void* y, int B, int Cin, int Cout, int Cp, int T,
                                 int H, int W, int k, void* workspace, hipStream_t s, int32_t* idx,
                                 const FsqParams* fsq) {
    const long long P = (long long)B * T * H * W;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipError_t e;
    if (idx && (!proj_fused(k, Cout, Cp, (long long)H * W, w_t != nullptr) || Cp > 8)) {
        // the unfused route: the latent (into y, or the workspace's last buffer), then FSQ
        const size_t base = conv_proj_workspace_bytes(B, Cin, Cout, Cp, T, H, W, k, w_s != nullptr, w_t != nullptr);
        void* lat = y ? y : static_cast<void*>(ws + base);
        if ((e = launch_conv_fact_proj(x, w_s, w_t, b_s, b_t, w_p, b_p, lat, B, Cin, Cout, Cp, T, H, W, k, ws, s)) !=
            hipSuccess)
            return e;
        return launch_fsq_quantize(lat, CVT_BF16, CVT_NTHWC, idx, nullptr, *fsq, B, (long long)T * H * W, s);
    }
    if (!proj_fused(k, Cout, Cp, (long long)H * W, w_t != nullptr)) {
        // conv into the workspace, then the 1x1 projection
        size_t off = conv_workspace_bytes(B, Cin, Cout, T, H, W, k, w_s != nullptr, w_t != nullptr);
        uint16_t* ymid = reinterpret_cast<uint16_t*>(ws + off);
        off += align256((size_t)P * Cout * 2);
        if ((e = launch_conv_fact(x, w_s, w_t, b_s, b_t, ymid, B, Cin, Cout, T, H, W, k, ws, s)) != hipSuccess)
            return e;
        return launch_conv_fact(ymid, w_p, nullptr, b_p, nullptr, y, B, Cout, Cp, T, H, W, 1, ws + off, s);
    }
    size_t off = 0;
    const uint16_t* tin = static_cast<const uint16_t*>(x);
    if (w_s) {  // spatial part on its own into the workspace
        uint8_t* sws = ws + off;
        off += pack_bytes(Cout, Cin, k * k);
        uint16_t* S = reinterpret_cast<uint16_t*>(ws + off);
        off += align256((size_t)P * Cout * 2);
        if ((e = launch_conv_fact(x, w_s, nullptr, b_s, nullptr, S, B, Cin, Cout, T, H, W, k, sws, s)) != hipSuccess)
            return e;
        tin = S;
    }
    uint16_t* wpt = reinterpret_cast<uint16_t*>(ws + off);
    off += pack_bytes(Cout, Cout, k);
    uint16_t* wpp = reinterpret_cast<uint16_t*>(ws + off);
    if ((e = pack_frag(w_t, wpt, Cout, Cout, 3, s)) != hipSuccess) return e;
    if ((e = pack_frag(w_p, wpp, Cp, Cout, 1, s)) != hipSuccess) return e;
    ConvGeom g{};
    g.P = P; g.T = T; g.H = H; g.W = W; g.Cin = Cout; g.Cout = Cout;
    g.kchunks = (Cout + BK - 1) / BK;
    RowsAux aux{};
    if (idx) {
        aux.fsq_idx = idx;
        aux.fsq = *fsq;
    }
    return launch_rows<TEMPORAL3>(tin, wpt, b_t, static_cast<uint16_t*>(y), g, B, s, wpp, b_p, Cp, nullptr, aux);
}

// Weights packed once by the caller (cvt_conv_weights_pack) for repeated calls: the order in
// which conv_rows_kernel reads them (pack_frag_kernel).  The packed calls run the row-tiled
// kernels only, with the caller's packed weights in place of the per-call repack; the
// results are those of the unpacked calls bit for bit (same kernels, same weights).
size_t conv_weights_packed_bytes(int Cout, int Cin, int taps) { return align256(frag_bytes(Cout, Cin, taps)); }

hipError_t launch_conv_weights_pack(const void* w, void* packed, int Cout, int Cin, int taps, hipStream_t s) {
    return pack_frag(w, static_cast<uint16_t*>(packed), Cout, Cin, taps, s);
}

bool conv_packed_supported(int Cin, int Cout, int H, int W, bool spatial, bool temporal) {
    return (!spatial || use_rows_kernel(3, Cout, rows_span_spatial(W), Cin)) &&
           (!temporal || use_rows_kernel(3, Cout, rows_span_temporal((long long)H * W), Cout));
}

size_t conv_packed_workspace_bytes(int B, int Cout, int T, int H, int W, bool spatial, bool temporal) {
    return spatial && temporal ? align256((size_t)B * T * H * W * Cout * 2) : 0;
}

hipError_t launch_conv_fact_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s,
                                   const float* b_t, void* y, int B, int Cin, int Cout, int T, int H, int W,
                                   void* workspace, hipStream_t s) {
    ConvGeom g{};
    g.P = (long long)B * T * H * W; g.T = T; g.H = H; g.W = W; g.Cin = Cin; g.Cout = Cout;
    g.kchunks = (Cin + BK - 1) / BK;
    const uint16_t* tin = static_cast<const uint16_t*>(x);
    hipError_t e;
    if (pw_s) {  // spatial part into the workspace (or y when there is no temporal part)
        uint16_t* sout = static_cast<uint16_t*>(pw_t ? workspace : y);
        if ((e = launch_rows<SPATIAL3>(tin, static_cast<const uint16_t*>(pw_s), b_s, sout, g, B, s)) != hipSuccess)
            return e;
        tin = sout;
    }
    if (!pw_t) return hipSuccess;
    g.Cin = Cout;
    g.kchunks = (Cout + BK - 1) / BK;
    return launch_rows<TEMPORAL3>(tin, static_cast<const uint16_t*>(pw_t), b_t, static_cast<uint16_t*>(y), g, B, s);
}

bool conv_proj_packed_supported(int Cin, int Cout, int Cp, int H, int W, bool spatial) {
    return proj_fused(3, Cout, Cp, (long long)H * W, true) &&
           (!spatial || use_rows_kernel(3, Cout, rows_span_spatial(W), Cin));
}

size_t conv_proj_packed_workspace_bytes(int B, int Cout, int T, int H, int W, bool spatial) {
    return spatial ? align256((size_t)B * T * H * W * Cout * 2) : 0;
}

hipError_t launch_conv_fact_proj_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s,
                                        const float* b_t, const void* pw_p, const float* b_p, void* y, int B, int Cin,
                                        int Cout, int Cp, int T, int H, int W, void* workspace, hipStream_t s) {
    const uint16_t* tin = static_cast<const uint16_t*>(x);
    hipError_t e;
    if (pw_s) {  // spatial part on its own into the workspace
        uint16_t* S = static_cast<uint16_t*>(workspace);
        if ((e = launch_conv_fact_packed(x, pw_s, nullptr, b_s, nullptr, S, B, Cin, Cout, T, H, W, nullptr, s)) !=
            hipSuccess)
            return e;
        tin = S;
    }
    ConvGeom g{};
    g.P = (long long)B * T * H * W; g.T = T; g.H = H; g.W = W; g.Cin = Cout; g.Cout = Cout;
    g.kchunks = (Cout + BK - 1) / BK;
    return launch_rows<TEMPORAL3>(tin, static_cast<const uint16_t*>(pw_t), b_t, static_cast<uint16_t*>(y), g, B, s,
                                  static_cast<const uint16_t*>(pw_p), b_p, Cp);
}

// Causal temporal convolution of one chunk of a stream (optionally with the fused 1x1
// projection): the frames before the chunk come from hist instead of the zero padding.
size_t conv_temporal_stream_workspace_bytes(int C, int Cp) {
    return pack_bytes(C, C, 3) + (Cp > 0 ? align256(frag_bytes(Cp, C, 1)) : 0);
}

bool conv_temporal_stream_supported(int C, int Cp, long long HW) {
    return use_rows_kernel(3, C, rows_span_temporal(HW), C) && (Cp == 0 || (C <= 256 && Cp <= 16));
}

hipError_t launch_conv_temporal_stream(const void* x, const void* hist, const void* w_t, const float* b_t,
                                       const void* w_p, const float* b_p, void* y, int B, int C, int Cp, int T,
                                       int H, int W, void* workspace, hipStream_t s) {
    const long long P = (long long)B * T * H * W;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* wpt = reinterpret_cast<uint16_t*>(ws);
    uint16_t* wpp = w_p ? reinterpret_cast<uint16_t*>(ws + pack_bytes(C, C, 3)) : nullptr;
    hipError_t e;
    if ((e = pack_frag(w_t, wpt, C, C, 3, s)) != hipSuccess) return e;
    if (w_p && (e = pack_frag(w_p, wpp, Cp, C, 1, s)) != hipSuccess) return e;
    ConvGeom g{};
    g.P = P; g.T = T; g.H = H; g.W = W; g.Cin = C; g.Cout = C;
    g.kchunks = (C + BK - 1) / BK;
    return launch_rows<TEMPORAL3>(static_cast<const uint16_t*>(x), wpt, b_t, static_cast<uint16_t*>(y), g, B, s, wpp,
                                  b_p, w_p ? Cp : 0, static_cast<const uint16_t*>(hist));
}

// ---------------------------------------------------------------------------------------------
// Encoder and decoder blocks.

// Residual block y = x + conv2(swish(LN2(conv1(swish(LN1(x)))))), conv = factorized causal
// conv C -> C, k = 3.  Workspace: the four packed weights and two bf16 [P][C] buffers A, S.
//   A = swish(LN1(x))                      (layernorm kernel)
//   S = spatial1(A)
//   A = swish(LN2(temporal1(S)))           (NORM epilogue; C > 256: plain conv + layernorm in place)
//   S = spatial2(A)
//   y = temporal2(S) + x                   (RES epilogue, one rounding)
bool resblock_supported(int C, int H, int W) {
    return use_rows_kernel(3, C, rows_span_spatial(W), C) && use_rows_kernel(3, C, rows_span_temporal((long long)H * W), C);
}

// packed: the four conv weights of w are already in the row kernels' fragment order
// (cvt_conv_weights_pack), so neither their workspace nor their repack is needed.
size_t resblock_workspace_bytes(int B, int C, int T, int H, int W, bool packed) {
    const size_t P = (size_t)B * T * H * W;
    return (packed ? 0 : 2 * pack_bytes(C, C, 9) + 2 * pack_bytes(C, C, 3)) + 2 * align256(P * C * 2);
}

hipError_t launch_resblock(const void* x, const cvt_resblock_weights& w, void* y, int B, int C, int T, int H, int W,
                           float eps, void* workspace, hipStream_t s, bool packed) {
    const long long P = (long long)B * T * H * W;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    size_t off = 0;
    auto take = [&](size_t n) {
        uint8_t* q = ws + off;
        off += n;
        return reinterpret_cast<uint16_t*>(q);
    };
    hipError_t e;
    const uint16_t *w1s, *w1t, *w2s, *w2t;
    if (packed) {
        w1s = static_cast<const uint16_t*>(w.c1_s);
        w1t = static_cast<const uint16_t*>(w.c1_t);
        w2s = static_cast<const uint16_t*>(w.c2_s);
        w2t = static_cast<const uint16_t*>(w.c2_t);
    } else {
        uint16_t* p1s = take(pack_bytes(C, C, 9));
        uint16_t* p1t = take(pack_bytes(C, C, 3));
        uint16_t* p2s = take(pack_bytes(C, C, 9));
        uint16_t* p2t = take(pack_bytes(C, C, 3));
        if ((e = pack_frag(w.c1_s, p1s, C, C, 9, s)) != hipSuccess) return e;
        if ((e = pack_frag(w.c1_t, p1t, C, C, 3, s)) != hipSuccess) return e;
        if ((e = pack_frag(w.c2_s, p2s, C, C, 9, s)) != hipSuccess) return e;
        if ((e = pack_frag(w.c2_t, p2t, C, C, 3, s)) != hipSuccess) return e;
        w1s = p1s; w1t = p1t; w2s = p2s; w2t = p2t;
    }
    uint16_t* A = take(align256((size_t)P * C * 2));
    uint16_t* S = take(align256((size_t)P * C * 2));
    ConvGeom g{};
    g.P = P; g.T = T; g.H = H; g.W = W; g.Cin = C; g.Cout = C;
    g.kchunks = (C + BK - 1) / BK;
    if ((e = launch_layernorm(x, w.ln1_g, w.ln1_b, A, P, C, eps, 1, s)) != hipSuccess) return e;
    if ((e = launch_rows<SPATIAL3>(A, w1s, w.c1_bs, S, g, B, s)) != hipSuccess) return e;
    if (C <= ROWS_NORM_MAX_C) {
        RowsAux aux{};
        aux.ln_g = w.ln2_g; aux.ln_b = w.ln2_b; aux.eps = eps; aux.swish = 1;
        if ((e = launch_rows<TEMPORAL3>(S, w1t, w.c1_bt, A, g, B, s, nullptr, nullptr, 0, nullptr, aux)) != hipSuccess)
            return e;
    } else {
        if ((e = launch_rows<TEMPORAL3>(S, w1t, w.c1_bt, A, g, B, s)) != hipSuccess) return e;
        if ((e = launch_layernorm(A, w.ln2_g, w.ln2_b, A, P, C, eps, 1, s)) != hipSuccess) return e;
    }
    if ((e = launch_rows<SPATIAL3>(A, w2s, w.c2_bs, S, g, B, s)) != hipSuccess) return e;
    RowsAux res{};
    res.res = static_cast<const uint16_t*>(x);
    return launch_rows<TEMPORAL3>(S, w2t, w.c2_bt, static_cast<uint16_t*>(y), g, B, s, nullptr, nullptr, 0, nullptr,
                                  res);
}

// Downsampling block: the spatial 1x3x3 conv at stride 2 in H and W (zero padding 1), then
// the causal temporal 3x1x1 conv at stride 2 (T = 1 + 2k -> 1 + k), either part optional, on
// conv_rows_kernel at stride 2 (conv_igemm_kernel with the strided input mapping for the
// shapes the row kernel does not take).
// packed: w_s and w_t hold the packed forms (cvt_conv_weights_pack), which only the row-tiled
// kernels read: both parts must take them (downsample_packed_supported), and the workspace
// holds only the intermediate.
bool downsample_packed_supported(int Cin, int Cout, int H, int W, bool space, bool time) {
    const int C1 = space ? Cout : Cin, H1 = space ? H / 2 : H, W1 = space ? W / 2 : W;
    return (!space || use_rows_kernel(3, Cout, rows_span_spatial(W), Cin)) &&
           (!time || (C1 == Cout && use_rows_kernel(3, Cout, rows_span_temporal((long long)H1 * W1), C1)));
}

size_t downsample_workspace_bytes(int B, int Cin, int Cout, int T, int H, int W, bool space, bool time, bool packed) {
    size_t b = 0;
    if (space && !packed) b += pack_bytes(Cout, Cin, 9);
    if (time && !packed) b += pack_bytes(Cout, space ? Cout : Cin, 3);
    if (space && time) b += align256((size_t)B * T * (H / 2) * (W / 2) * Cout * 2);
    return b;
}

hipError_t launch_downsample(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                             void* y, int B, int Cin, int Cout, int T, int H, int W, void* workspace, hipStream_t s,
                             bool packed) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    // workspace: [spatial weights][temporal weights] (repacked per call only) [intermediate]
    const size_t ps = w_s && !packed ? pack_bytes(Cout, Cin, 9) : 0;
    const size_t pt = w_t && !packed ? pack_bytes(Cout, w_s ? Cout : Cin, 3) : 0;
    hipError_t e;
    const uint16_t* tin = static_cast<const uint16_t*>(x);
    int C1 = Cin, H1 = H, W1 = W;
    if (w_s) {
        uint16_t* pbuf = reinterpret_cast<uint16_t*>(ws);  // per-call repack target
        const uint16_t* wps = packed ? static_cast<const uint16_t*>(w_s) : pbuf;
        uint16_t* S = w_t ? reinterpret_cast<uint16_t*>(ws + ps + pt) : static_cast<uint16_t*>(y);
        H1 = H / 2;
        W1 = W / 2;
        ConvGeom g{};
        g.P = (long long)B * T * H1 * W1; g.T = T; g.H = H1; g.W = W1; g.Cin = Cin; g.Cout = Cout;
        g.kchunks = (Cin + BK - 1) / BK;
        g.Ti = T; g.Hi = H; g.Wi = W; g.st = 1; g.ss = 2;
        if (use_rows_kernel(3, Cout, rows_span_spatial(W), Cin)) {
            if (!packed && (e = pack_frag(w_s, pbuf, Cout, Cin, 9, s)) != hipSuccess) return e;
            if ((e = launch_rows_s2<SPATIAL3>(tin, wps, b_s, S, g, B, s)) != hipSuccess) return e;
        } else {
            if (packed) return hipErrorInvalidValue;
            if ((e = pack(w_s, pbuf, Cout, Cin, 9, s)) != hipSuccess) return e;
            if ((e = launch_igemm(SPATIAL3, tin, wps, b_s, S, g, s)) != hipSuccess) return e;
        }
        tin = S;
        C1 = Cout;
    }
    if (!w_t) return hipSuccess;
    uint16_t* pbuf = reinterpret_cast<uint16_t*>(ws + ps);  // per-call repack target
    const uint16_t* wpt = packed ? static_cast<const uint16_t*>(w_t) : pbuf;
    const int T1 = 1 + (T - 1) / 2;
    ConvGeom g{};
    g.P = (long long)B * T1 * H1 * W1; g.T = T1; g.H = H1; g.W = W1; g.Cin = C1; g.Cout = Cout;
    g.kchunks = (C1 + BK - 1) / BK;
    g.Ti = T; g.Hi = H1; g.Wi = W1; g.st = 2; g.ss = 1;
    if (C1 == Cout && use_rows_kernel(3, Cout, rows_span_temporal((long long)H1 * W1), C1)) {
        if (!packed && (e = pack_frag(w_t, pbuf, Cout, C1, 3, s)) != hipSuccess) return e;
        return launch_rows_s2<TEMPORAL3>(tin, wpt, b_t, static_cast<uint16_t*>(y), g, B, s);
    }
    if (packed) return hipErrorInvalidValue;
    if ((e = pack(w_t, pbuf, Cout, C1, 3, s)) != hipSuccess) return e;
    return launch_igemm(TEMPORAL3, tin, wpt, b_t, static_cast<uint16_t*>(y), g, s);
}

// Decoder upsampling block: nearest-neighbour repetition (x2 in H and W and/or causal x2 in
// time, T -> 2T - 1) followed by the factorized conv, with the repetition done by the conv's
// region loads (conv_rows_kernel reads the low-resolution input through the upsampled
// index), so the repeated tensor is never written.  The spatial conv runs on the T input
// frames (it is frame-local, so repeating frames before or after it is the same), the
// temporal conv reads those frames through the causal repetition.
bool upsample_supported(int Cin, int Cout, int W_in, long long HW_mid) {
    return use_rows_kernel(3, Cout, rows_span_spatial(W_in), Cin) &&
           use_rows_kernel(3, Cout, rows_span_temporal(HW_mid), Cout);
}

// packed: w_s and w_t hold the packed forms (cvt_conv_weights_pack); the workspace holds only
// the intermediate.
size_t upsample_workspace_bytes(int B, int Cin, int Cout, int T, int H, int W, bool up_space, bool packed) {
    const int f = up_space ? 2 : 1;
    return (packed ? 0 : pack_bytes(Cout, Cin, 9) + pack_bytes(Cout, Cout, 3)) +
           align256((size_t)B * T * (f * H) * (f * W) * Cout * 2);
}

hipError_t launch_upsample(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                           int B, int Cin, int Cout, int T, int H, int W, bool up_space, bool up_time, void* workspace,
                           hipStream_t s, bool packed) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const size_t pw = packed ? 0 : pack_bytes(Cout, Cin, 9) + pack_bytes(Cout, Cout, 3);
    uint16_t* ps_buf = reinterpret_cast<uint16_t*>(ws);  // per-call repack targets
    uint16_t* pt_buf = reinterpret_cast<uint16_t*>(ws + pack_bytes(Cout, Cin, 9));
    const uint16_t* wps = packed ? static_cast<const uint16_t*>(w_s) : ps_buf;
    const uint16_t* wpt = packed ? static_cast<const uint16_t*>(w_t) : pt_buf;
    uint16_t* S = reinterpret_cast<uint16_t*>(ws + pw);
    const int Ho = up_space ? 2 * H : H, Wo = up_space ? 2 * W : W, To = up_time ? 2 * T - 1 : T;
    hipError_t e;
    if (!packed) {
        if ((e = pack_frag(w_s, ps_buf, Cout, Cin, 9, s)) != hipSuccess) return e;
        if ((e = pack_frag(w_t, pt_buf, Cout, Cout, 3, s)) != hipSuccess) return e;
    }
    ConvGeom g{};
    g.P = (long long)B * T * Ho * Wo; g.T = T; g.H = Ho; g.W = Wo; g.Cin = Cin; g.Cout = Cout;
    g.kchunks = (Cin + BK - 1) / BK;
    g.ups = up_space ? 1 : 0; g.Ti = T; g.Hi = H; g.Wi = W;
    if ((e = launch_rows<SPATIAL3>(static_cast<const uint16_t*>(x), wps, b_s, S, g, B, s)) != hipSuccess) return e;
    ConvGeom g2{};
    g2.P = (long long)B * To * Ho * Wo; g2.T = To; g2.H = Ho; g2.W = Wo; g2.Cin = Cout; g2.Cout = Cout;
    g2.kchunks = (Cout + BK - 1) / BK;
    g2.ups = up_time ? 1 : 0; g2.Ti = T; g2.Hi = Ho; g2.Wi = Wo;
    return launch_rows<TEMPORAL3>(S, wpt, b_t, static_cast<uint16_t*>(y), g2, B, s);
}

hipError_t launch_fsq_dequant_proj(const int32_t* idx, const FsqParams& p, const void* w_p, const float* b_p, void* y,
                                   long long P, int Cout, int32_t* invalid, hipStream_t s) {
    const int ng = (Cout + 7) / 8;
    const dim3 grid((unsigned)small_proj_blocks(P * ng, ng));
    const bool def = p.D == 6 && p.levels[0] == 8 && p.levels[1] == 8 && p.levels[2] == 8 && p.levels[3] == 5 &&
                     p.levels[4] == 5 && p.levels[5] == 5;
    if (def && small_proj_staged(p.D, Cout))
        hipLaunchKernelGGL((fsq_dequant_proj_kernel<8, true>), grid, dim3(256), small_proj_lds(p.D, Cout), s, idx, p,
                           static_cast<const uint16_t*>(w_p), b_p, static_cast<uint16_t*>(y), P, Cout, invalid);
    else if (small_proj_staged(p.D, Cout))  // D <= 8
        hipLaunchKernelGGL(fsq_dequant_proj_kernel<8>, grid, dim3(256), small_proj_lds(p.D, Cout), s, idx, p,
                           static_cast<const uint16_t*>(w_p), b_p, static_cast<uint16_t*>(y), P, Cout, invalid);
    else
        hipLaunchKernelGGL(fsq_dequant_proj_kernel<0>, grid, dim3(256), 0, s, idx, p,
                           static_cast<const uint16_t*>(w_p), b_p, static_cast<uint16_t*>(y), P, Cout, invalid);
    return hipGetLastError();
}

}  // namespace cvt
