// C ABI entry points: argument validation, host-side parameter preparation
// and dispatch to the HIP launchers.  Every check runs before any launch, so
// an error status means nothing was enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <limits>

#include "cvt_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return CVT_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CVT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int d) { return d == CVT_F32 || d == CVT_BF16; }
bool valid_layout(int l) { return l == CVT_NCTHW || l == CVT_NTHWC; }

int check_window(const void* a, const void* b, int dtype, int B, int C, int T, int H, int W, int t0, int nt, int Tp,
                 int Hp, int Wp, long long frames) {
    if (!a || !b) return fail(CVT_E_NULL, "null tensor pointer");
    if (!valid_dtype(dtype)) return fail(CVT_E_DTYPE, "dtype must be CVT_F32 or CVT_BF16");
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0 || nt <= 0 || Tp <= 0 || Hp <= 0 || Wp <= 0)
        return fail(CVT_E_SHAPE, "non-positive size");
    if (t0 < 0 || (long long)t0 + nt > T)
        return fail(CVT_E_SHAPE, "window %d + %d outside the clip of %d frames", t0, nt, T);
    if (Tp < nt || Hp < H || Wp < W)
        return fail(CVT_E_SHAPE, "padded size %dx%dx%d below the window's %dx%dx%d", Tp, Hp, Wp, nt, H, W);
    if ((long long)Hp * Wp >= (1LL << 30)) return fail(CVT_E_SHAPE, "a padded frame of Hp*Wp must stay below 2^30");
    if ((long long)B * C * frames >= (1LL << 31)) return fail(CVT_E_SHAPE, "B*C*Tp must stay below 2^31");
    if (!aligned16(a) || !aligned16(b)) return fail(CVT_E_ALIGN, "tensor pointers must be 16-byte aligned");
    return CVT_OK;
}

int check_haar(const void* a, int a_dt, const void* b, int b_dt, int layout, int B, int C, int T, int H, int W,
               int tl) {
    if (!a || !b) return fail(CVT_E_NULL, "null tensor pointer");
    if (!valid_dtype(a_dt) || !valid_dtype(b_dt)) return fail(CVT_E_DTYPE, "dtype must be CVT_F32 or CVT_BF16");
    if (!valid_layout(layout)) return fail(CVT_E_LAYOUT, "layout must be CVT_NCTHW or CVT_NTHWC");
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (tl != 0 && tl != 2 && tl != 3) return fail(CVT_E_SHAPE, "temporal_levels must be 0, 2 or 3, got %d", tl);
    if (H % 4 || W % 4) return fail(CVT_E_SHAPE, "H and W must be multiples of 4 (got %dx%d)", H, W);
    if (tl == 2 && (T - 1) % 4) return fail(CVT_E_SHAPE, "temporal Haar needs T = 1 + 4k frames (got %d)", T);
    if (tl == 3 && T % 4) return fail(CVT_E_SHAPE, "a continuation chunk needs T = 4k frames (got %d)", T);
    if (!aligned16(a) || !aligned16(b)) return fail(CVT_E_ALIGN, "tensor pointers must be 16-byte aligned");
    return CVT_OK;
}

// pix: the clip, coef: the padded window's coefficients.
int check_haar_window(const void* pix, int pix_dt, const void* coef, int coef_dt, int layout, int B, int C, int T,
                      int H, int W, int t0, int nt, int Tp, int Hp, int Wp, int tl) {
    if (tl == 3) return fail(CVT_E_SHAPE, "a window starts with its own causal first frame: temporal_levels 0 or 2");
    int st = check_haar(coef, coef_dt, pix, pix_dt, layout, B, C, Tp, Hp, Wp, tl);
    if (st != CVT_OK) return st;
    return check_window(pix, coef, pix_dt, B, C, T, H, W, t0, nt, Tp, Hp, Wp, Tp);
}

// FSQ breakpoints.  For L levels with h = (L-1)(1+eps)/2, o = 1/2 (L even) or
// 0, s = atanh(o/h), the rounded bound q = rint(tanh(z+s) h - o) steps from j
// to j+1 where tanh(z+s) h - o = j + 1/2, i.e. at z_j = atanh((j+1/2+o)/h) - s,
// j = -floor(L/2) .. ceil(L/2) - 2 (L - 1 breakpoints).  The digit
// d = q + floor(L/2) is the number of breakpoints below z.  Each z_j is
// replaced by the smallest float f with f > z_j, so that for every float z
// "z >= f" is exactly "z > z_j".
constexpr double kFsqEps = 1e-3;

float float_above(double zj) {
    float f = (float)zj;
    if ((double)f <= zj) f = nextafterf(f, std::numeric_limits<float>::infinity());
    return f;
}

int fsq_params(const int32_t* levels, int D, cvt::FsqParams* p) {
    if (!levels) return fail(CVT_E_NULL, "levels is NULL");
    if (D < 1 || D > cvt::FSQ_MAX_D) return fail(CVT_E_LEVELS, "D must be in [1, %d], got %d", cvt::FSQ_MAX_D, D);
    memset(p, 0, sizeof(*p));
    p->D = D;
    long long prod = 1;
    for (int i = 0; i < D; ++i) {
        const int L = levels[i];
        if (L < 2 || L > cvt::FSQ_MAX_L)
            return fail(CVT_E_LEVELS, "level %d is %d, must be in [2, %d]", i, L, cvt::FSQ_MAX_L);
        p->levels[i] = L;
        p->basis[i] = (int)prod;
        prod *= L;
        if (prod >= (1LL << 31)) return fail(CVT_E_LEVELS, "product of levels must be below 2^31");
        p->half[i] = L / 2;
        p->nthr[i] = L - 1;
        int l = 0;
        while ((1 << l) < L) ++l;
        p->magic[i] = (unsigned int)(((1ull << (31 + l)) + (unsigned long long)L - 1ull) / (unsigned long long)L);
        p->shift[i] = l - 1;
        const double h = (L - 1) * (1.0 + kFsqEps) / 2.0;
        const double o = (L % 2 == 0) ? 0.5 : 0.0;
        const double s = atanh(o / h);
        const int half = L / 2;
        for (int j = 0; j < cvt::FSQ_MAX_L - 1; ++j) p->thr[i][j] = std::numeric_limits<float>::quiet_NaN();
        for (int j = -half, n = 0; j <= (L + 1) / 2 - 2; ++j, ++n) p->thr[i][n] = float_above(atanh((j + 0.5 + o) / h) - s);
    }
    p->codebook = (int)prod;
    return CVT_OK;
}

}  // namespace

extern "C" {

int cvt_abi_version(void) { return 1; }

const char* cvt_status_string(int s) {
    switch (s) {
        case CVT_OK: return "CVT_OK";
        case CVT_E_NULL: return "CVT_E_NULL: a required pointer is NULL";
        case CVT_E_SHAPE: return "CVT_E_SHAPE: invalid size or shape";
        case CVT_E_DTYPE: return "CVT_E_DTYPE: unsupported dtype";
        case CVT_E_LAYOUT: return "CVT_E_LAYOUT: unsupported layout";
        case CVT_E_ALIGN: return "CVT_E_ALIGN: pointer not 16-byte aligned";
        case CVT_E_LEVELS: return "CVT_E_LEVELS: unsupported FSQ levels";
        case CVT_E_WORKSPACE: return "CVT_E_WORKSPACE: workspace missing or too small";
        case CVT_E_HIP: return "CVT_E_HIP: HIP runtime error";
        default: return "unknown cvt status";
    }
}

const char* cvt_last_error(void) { return g_err; }

int cvt_haar3d_fwd(const void* x, int x_dtype, void* y, int y_dtype, int y_layout, int B, int C, int T, int H, int W,
                   int temporal_levels, void* stream) {
    const int st = check_haar(x, x_dtype, y, y_dtype, y_layout, B, C, T, H, W, temporal_levels);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_haar_fwd(x, x_dtype, y, y_dtype, y_layout, B, C, T, H, W, temporal_levels,
                                           (hipStream_t)stream),
                      "cvt_haar3d_fwd launch");
}

int cvt_haar3d_inv(const void* y, int y_dtype, int y_layout, void* x, int x_dtype, int B, int C, int T, int H, int W,
                   int temporal_levels, void* stream) {
    const int st = check_haar(y, y_dtype, x, x_dtype, y_layout, B, C, T, H, W, temporal_levels);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_haar_inv(y, y_dtype, y_layout, x, x_dtype, B, C, T, H, W, temporal_levels,
                                           (hipStream_t)stream),
                      "cvt_haar3d_inv launch");
}

size_t cvt_causal_conv3d_fact_workspace(int B, int Cin, int Cout, int T, int H, int W, int k, int parts) {
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0 || (k != 1 && k != 3)) return 0;
    if (parts < 1 || parts > 3) return 0;
    return cvt::conv_workspace_bytes(B, Cin, Cout, T, H, W, k, (parts & CVT_CONV_SPATIAL) != 0,
                                     (parts & CVT_CONV_TEMPORAL) != 0);
}

namespace {
// The checks of cvt_causal_conv3d_fact that do not concern the workspace.
int check_conv_fact(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                    int B, int Cin, int Cout, int T, int H, int W, int k) {
    if (!x || !y) return fail(CVT_E_NULL, "x and y must not be NULL");
    if (!w_s && !w_t) return fail(CVT_E_NULL, "at least one of w_s and w_t must be given");
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0)
        return fail(CVT_E_SHAPE, "non-positive size");
    if (k != 1 && k != 3) return fail(CVT_E_SHAPE, "k must be 1 or 3, got %d", k);
    if (Cout > 4096) return fail(CVT_E_SHAPE, "Cout must be at most 4096, got %d", Cout);
    if (!w_s && Cin != Cout)
        return fail(CVT_E_SHAPE, "a temporal-only call needs Cin == Cout (got %d and %d)", Cin, Cout);
    if (Cin % 8 != 0 && !(k == 1 && Cin <= 16 && w_s))
        return fail(CVT_E_SHAPE, "Cin must be a multiple of 8 (or at most 16 with k = 1), got %d", Cin);
    if (w_t && Cout % 8 != 0)
        return fail(CVT_E_SHAPE, "the temporal convolution needs Cout to be a multiple of 8, got %d", Cout);
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_s) & 1u) || (reinterpret_cast<uintptr_t>(w_t) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    return CVT_OK;
}
}  // namespace

int cvt_causal_conv3d_fact(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                           void* y, int B, int Cin, int Cout, int T, int H, int W, int k, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const int st = check_conv_fact(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, k);
    if (st != CVT_OK) return st;
    const size_t need = cvt::conv_workspace_bytes(B, Cin, Cout, T, H, W, k, w_s != nullptr, w_t != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(cvt::launch_conv_fact(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, k, workspace,
                                            (hipStream_t)stream),
                      "cvt_causal_conv3d_fact launch");
}

int cvt_causal_conv3d_fact_noalloc(const void* x, const void* w_s, const void* w_t, const float* b_s,
                                   const float* b_t, void* y, int B, int Cin, int Cout, int T, int H, int W, int k,
                                   void* stream) {
    const int st = check_conv_fact(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, k);
    if (st != CVT_OK) return st;
    const size_t need = cvt::conv_workspace_bytes(B, Cin, Cout, T, H, W, k, w_s != nullptr, w_t != nullptr);
    if (need > CVT_NOALLOC_SCRATCH_BYTES)
        return fail(CVT_E_WORKSPACE,
                    "this call needs %zu bytes of scratch; the library's preallocated scratch holds %zu "
                    "(use cvt_causal_conv3d_fact with a caller workspace)",
                    need, (size_t)CVT_NOALLOC_SCRATCH_BYTES);
    return hip_status(cvt::launch_conv_fact_noalloc(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, k,
                                                    (hipStream_t)stream),
                      "cvt_causal_conv3d_fact_noalloc launch");
}

size_t cvt_conv_weights_packed_bytes(int Cout, int Cin, int taps) {
    if (Cout <= 0 || Cin <= 0 || Cout > 4096 || Cin > 4096 || (taps != 1 && taps != 3 && taps != 9)) return 0;
    return cvt::conv_weights_packed_bytes(Cout, Cin, taps);
}

int cvt_conv_weights_pack(const void* w, void* packed, int Cout, int Cin, int taps, void* stream) {
    if (!w || !packed) return fail(CVT_E_NULL, "w and packed must not be NULL");
    if (Cout <= 0 || Cin <= 0 || Cout > 4096 || Cin > 4096)
        return fail(CVT_E_SHAPE, "Cout and Cin must be in 1..4096, got %d and %d", Cout, Cin);
    if (taps != 1 && taps != 3 && taps != 9) return fail(CVT_E_SHAPE, "taps must be 1, 3 or 9, got %d", taps);
    if (reinterpret_cast<uintptr_t>(w) & 1u) return fail(CVT_E_ALIGN, "w must be 2-byte aligned");
    if (!aligned16(packed)) return fail(CVT_E_ALIGN, "packed must be 16-byte aligned");
    return hip_status(cvt::launch_conv_weights_pack(w, packed, Cout, Cin, taps, (hipStream_t)stream),
                      "cvt_conv_weights_pack launch");
}

size_t cvt_causal_conv3d_fact_packed_workspace(int B, int Cout, int T, int H, int W, int parts) {
    if (B <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0 || parts < 1 || parts > 3) return 0;
    return cvt::conv_packed_workspace_bytes(B, Cout, T, H, W, (parts & CVT_CONV_SPATIAL) != 0,
                                            (parts & CVT_CONV_TEMPORAL) != 0);
}

namespace {
// The checks shared by the two packed-weight calls (the projection's own ones aside).
int check_conv_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s, const float* b_t, void* y,
                      int B, int Cin, int Cout, int T, int H, int W) {
    if (!x || !y) return fail(CVT_E_NULL, "x and y must not be NULL");
    if (!pw_s && !pw_t) return fail(CVT_E_NULL, "at least one of pw_s and pw_t must be given");
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (Cout > 4096) return fail(CVT_E_SHAPE, "Cout must be at most 4096, got %d", Cout);
    if (!pw_s && Cin != Cout)
        return fail(CVT_E_SHAPE, "a temporal-only call needs Cin == Cout (got %d and %d)", Cin, Cout);
    if (Cin % 8 != 0 || Cout % 8 != 0)
        return fail(CVT_E_SHAPE, "packed weights need Cin and Cout to be multiples of 8, got %d and %d", Cin, Cout);
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    if ((pw_s && !aligned16(pw_s)) || (pw_t && !aligned16(pw_t)))
        return fail(CVT_E_ALIGN, "packed weights must be 16-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    return CVT_OK;
}

int check_packed_workspace(void* workspace, size_t workspace_bytes, size_t need) {
    if (need == 0) return CVT_OK;
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return CVT_OK;
}
}  // namespace

int cvt_causal_conv3d_fact_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s, const float* b_t,
                                  void* y, int B, int Cin, int Cout, int T, int H, int W, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    int st = check_conv_packed(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W);
    if (st != CVT_OK) return st;
    if (Cout < 64 || !cvt::conv_packed_supported(Cin, Cout, H, W, pw_s != nullptr, pw_t != nullptr))
        return fail(CVT_E_SHAPE, "packed weights run the row-tiled kernels: Cout >= 64 and a tile's rows of the "
                                 "input (10 image rows, 9 frames) below 2 GiB (Cin=%d, Cout=%d)", Cin, Cout);
    const size_t need = cvt::conv_packed_workspace_bytes(B, Cout, T, H, W, pw_s != nullptr, pw_t != nullptr);
    if ((st = check_packed_workspace(workspace, workspace_bytes, need)) != CVT_OK) return st;
    return hip_status(cvt::launch_conv_fact_packed(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W, workspace,
                                                   (hipStream_t)stream),
                      "cvt_causal_conv3d_fact_packed launch");
}

size_t cvt_causal_conv3d_fact_proj_packed_workspace(int B, int Cout, int T, int H, int W, int parts) {
    if (B <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0 || parts < 2 || parts > 3) return 0;
    return cvt::conv_proj_packed_workspace_bytes(B, Cout, T, H, W, (parts & CVT_CONV_SPATIAL) != 0);
}

int cvt_causal_conv3d_fact_proj_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s,
                                       const float* b_t, const void* pw_p, const float* b_p, void* y, int B, int Cin,
                                       int Cout, int Cp, int T, int H, int W, void* workspace, size_t workspace_bytes,
                                       void* stream) {
    if (!pw_t || !pw_p) return fail(CVT_E_NULL, "pw_t and pw_p must not be NULL (the projection runs in the "
                                                "temporal convolution's epilogue)");
    int st = check_conv_packed(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W);
    if (st != CVT_OK) return st;
    if (Cp < 1 || Cp > 16 || Cout > 256)
        return fail(CVT_E_SHAPE, "the fused projection needs Cout <= 256 and 1 <= Cp <= 16 (got Cout=%d, Cp=%d)", Cout,
                    Cp);
    if (Cout < 64 || !cvt::conv_proj_packed_supported(Cin, Cout, Cp, H, W, pw_s != nullptr))
        return fail(CVT_E_SHAPE, "packed weights run the row-tiled kernels: Cout >= 64 and a tile's rows of the "
                                 "input (10 image rows, 9 frames) below 2 GiB (Cin=%d, Cout=%d)", Cin, Cout);
    if (!aligned16(pw_p)) return fail(CVT_E_ALIGN, "packed weights must be 16-byte aligned");
    if (b_p && (reinterpret_cast<uintptr_t>(b_p) & 3u)) return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::conv_proj_packed_workspace_bytes(B, Cout, T, H, W, pw_s != nullptr);
    if ((st = check_packed_workspace(workspace, workspace_bytes, need)) != CVT_OK) return st;
    return hip_status(cvt::launch_conv_fact_proj_packed(x, pw_s, pw_t, b_s, b_t, pw_p, b_p, y, B, Cin, Cout, Cp, T, H,
                                                        W, workspace, (hipStream_t)stream),
                      "cvt_causal_conv3d_fact_proj_packed launch");
}

size_t cvt_causal_conv3d_fact_proj_workspace(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k, int parts) {
    if (B <= 0 || Cin <= 0 || Cout <= 0 || Cp <= 0 || T <= 0 || H <= 0 || W <= 0 || (k != 1 && k != 3)) return 0;
    if (parts < 1 || parts > 3) return 0;
    return cvt::conv_proj_workspace_bytes(B, Cin, Cout, Cp, T, H, W, k, (parts & CVT_CONV_SPATIAL) != 0,
                                          (parts & CVT_CONV_TEMPORAL) != 0);
}

int cvt_causal_conv3d_fact_proj(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                                const void* w_p, const float* b_p, void* y, int B, int Cin, int Cout, int Cp, int T,
                                int H, int W, int k, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !y || !w_p) return fail(CVT_E_NULL, "x, w_p and y must not be NULL");
    if (!w_s && !w_t) return fail(CVT_E_NULL, "at least one of w_s and w_t must be given");
    if (B <= 0 || Cin <= 0 || Cout <= 0 || Cp <= 0 || T <= 0 || H <= 0 || W <= 0)
        return fail(CVT_E_SHAPE, "non-positive size");
    if (k != 1 && k != 3) return fail(CVT_E_SHAPE, "k must be 1 or 3, got %d", k);
    if (Cout > 4096 || Cp > 4096) return fail(CVT_E_SHAPE, "Cout and Cp must be at most 4096, got %d and %d", Cout, Cp);
    if (!w_s && Cin != Cout)
        return fail(CVT_E_SHAPE, "a temporal-only call needs Cin == Cout (got %d and %d)", Cin, Cout);
    if (Cin % 8 != 0) return fail(CVT_E_SHAPE, "Cin must be a multiple of 8, got %d", Cin);
    if (Cout % 8 != 0) return fail(CVT_E_SHAPE, "Cout must be a multiple of 8, got %d", Cout);
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_s) & 1u) || (reinterpret_cast<uintptr_t>(w_t) & 1u) ||
        (reinterpret_cast<uintptr_t>(w_p) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)) ||
        (b_p && (reinterpret_cast<uintptr_t>(b_p) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need =
        cvt::conv_proj_workspace_bytes(B, Cin, Cout, Cp, T, H, W, k, w_s != nullptr, w_t != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(cvt::launch_conv_fact_proj(x, w_s, w_t, b_s, b_t, w_p, b_p, y, B, Cin, Cout, Cp, T, H, W, k,
                                                 workspace, (hipStream_t)stream),
                      "cvt_causal_conv3d_fact_proj launch");
}

size_t cvt_causal_conv3d_temporal_stream_workspace(int C, int Cp) {
    if (C <= 0 || Cp < 0) return 0;
    return cvt::conv_temporal_stream_workspace_bytes(C, Cp);
}

int cvt_causal_conv3d_temporal_stream(const void* x, const void* hist, const void* w_t, const float* b_t,
                                      const void* w_p, const float* b_p, void* y, int B, int C, int Cp, int T, int H,
                                      int W, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !w_t || !y) return fail(CVT_E_NULL, "x, w_t and y must not be NULL");
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    const int cp = w_p ? Cp : 0;
    if (w_p && (Cp < 1 || Cp > 16 || C > 256))
        return fail(CVT_E_SHAPE, "the fused projection needs C <= 256 and 1 <= Cp <= 16 (got C=%d, Cp=%d)", C, Cp);
    // a tile's frames (and the two history frames) are addressed with 31-bit byte offsets
    if (C < 64 || C % 8 != 0 || !cvt::conv_temporal_stream_supported(C, cp, (long long)H * W))
        return fail(CVT_E_SHAPE, "the stream convolution needs C >= 64, C %% 8 == 0 and 9 frames of the input below "
                                 "2 GiB (C=%d)", C);
    if (!aligned16(x) || !aligned16(y) || (hist && !aligned16(hist)))
        return fail(CVT_E_ALIGN, "x, hist and y must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_t) & 1u) || (reinterpret_cast<uintptr_t>(w_p) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)) || (b_p && (reinterpret_cast<uintptr_t>(b_p) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::conv_temporal_stream_workspace_bytes(C, cp);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(cvt::launch_conv_temporal_stream(x, hist, w_t, b_t, w_p, b_p, y, B, C, cp, T, H, W, workspace,
                                                       (hipStream_t)stream),
                      "cvt_causal_conv3d_temporal_stream launch");
}

int cvt_attention3d(const void* q, const void* k, const void* v, void* out, int B, int C, int T, int H, int W,
                    int heads, int axis, void* stream) {
    if (!q || !k || !v || !out) return fail(CVT_E_NULL, "q, k, v and out must not be NULL");
    if (axis != CVT_ATTN_SPATIAL && axis != CVT_ATTN_TEMPORAL_CAUSAL)
        return fail(CVT_E_LAYOUT, "axis must be CVT_ATTN_SPATIAL or CVT_ATTN_TEMPORAL_CAUSAL, got %d", axis);
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0 || heads <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (C % 8 != 0 || C > 4096) return fail(CVT_E_SHAPE, "C must be a multiple of 8 and at most 4096, got %d", C);
    if (C % heads != 0) return fail(CVT_E_SHAPE, "heads (%d) must divide C (%d)", heads, C);
    const int d = C / heads;
    if (d % 8 != 0 || d > 256) return fail(CVT_E_SHAPE, "the head dim must be a multiple of 8 up to 256, got %d", d);
    if ((long long)H * W * C >= (1LL << 30)) return fail(CVT_E_SHAPE, "a frame of H * W * C must stay below 2^30");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(CVT_E_ALIGN, "tensor pointers must be 16-byte aligned");
    return hip_status(cvt::launch_attention3d(q, k, v, out, B, C, T, H, W, heads, axis, (hipStream_t)stream),
                      "cvt_attention3d launch");
}

int cvt_fsq_quantize(const void* z, int z_dtype, int z_layout, int32_t* indices, void* codes, const int32_t* levels,
                     int D, int B, int T, int H, int W, void* stream) {
    if (!z || !indices) return fail(CVT_E_NULL, "z and indices must not be NULL");
    if (!valid_dtype(z_dtype)) return fail(CVT_E_DTYPE, "dtype must be CVT_F32 or CVT_BF16");
    if (!valid_layout(z_layout)) return fail(CVT_E_LAYOUT, "layout must be CVT_NCTHW or CVT_NTHWC");
    if (B <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    cvt::FsqParams p;
    const int st = fsq_params(levels, D, &p);
    if (st != CVT_OK) return st;
    if (!aligned16(z) || !aligned16(indices) || (codes && !aligned16(codes)))
        return fail(CVT_E_ALIGN, "tensor pointers must be 16-byte aligned");
    const long long npb = (long long)T * H * W;
    return hip_status(cvt::launch_fsq_quantize(z, z_dtype, z_layout, indices, codes, p, B, npb, (hipStream_t)stream),
                      "cvt_fsq_quantize launch");
}

int cvt_fsq_dequantize(const int32_t* indices, void* codes, int c_dtype, int c_layout, const int32_t* levels, int D,
                       int B, int T, int H, int W, int32_t* d_invalid_count, void* stream) {
    if (!indices || !codes) return fail(CVT_E_NULL, "indices and codes must not be NULL");
    if (!valid_dtype(c_dtype)) return fail(CVT_E_DTYPE, "dtype must be CVT_F32 or CVT_BF16");
    if (!valid_layout(c_layout)) return fail(CVT_E_LAYOUT, "layout must be CVT_NCTHW or CVT_NTHWC");
    if (B <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    cvt::FsqParams p;
    const int st = fsq_params(levels, D, &p);
    if (st != CVT_OK) return st;
    if (!aligned16(indices) || !aligned16(codes)) return fail(CVT_E_ALIGN, "tensor pointers must be 16-byte aligned");
    if (d_invalid_count && (reinterpret_cast<uintptr_t>(d_invalid_count) & 3u))
        return fail(CVT_E_ALIGN, "the invalid-index counter must be 4-byte aligned");
    const long long npb = (long long)T * H * W;
    return hip_status(cvt::launch_fsq_dequantize(indices, codes, c_dtype, c_layout, p, B, npb, d_invalid_count,
                                                 (hipStream_t)stream),
                      "cvt_fsq_dequantize launch");
}

int cvt_video_window(int T, int H, int W, int window, int t_align, int s_align, int index, int* n_windows, int* t0,
                     int* nt, int* Tp, int* Hp, int* Wp) {
    if (T <= 0 || H <= 0 || W <= 0 || window <= 0 || t_align <= 0 || s_align <= 0)
        return fail(CVT_E_SHAPE, "sizes, window and alignments must be positive");
    const long long n = ((long long)T + window - 1) / window;
    if (index < 0 || index >= n) return fail(CVT_E_SHAPE, "window index %d outside [0, %lld)", index, n);
    const long long a = (long long)index * window;
    const long long len = std::min((long long)window, (long long)T - a);
    const long long tp = 1 + ((len - 1 + t_align - 1) / t_align) * t_align;
    const long long hp = ((long long)H + s_align - 1) / s_align * s_align;
    const long long wp = ((long long)W + s_align - 1) / s_align * s_align;
    const long long imax = std::numeric_limits<int>::max();
    if (tp > imax || hp > imax || wp > imax) return fail(CVT_E_SHAPE, "padded size above INT_MAX");
    if (n_windows) *n_windows = (int)n;
    if (t0) *t0 = (int)a;
    if (nt) *nt = (int)len;
    if (Tp) *Tp = (int)tp;
    if (Hp) *Hp = (int)hp;
    if (Wp) *Wp = (int)wp;
    return ok();
}


int cvt_video_pad(const void* x, void* y, int dtype, int B, int C, int T, int H, int W, int t0, int nt, int Tp, int Hp,
                  int Wp, void* stream) {
    const int st = check_window(x, y, dtype, B, C, T, H, W, t0, nt, Tp, Hp, Wp, Tp);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_video_pad(x, y, dtype, B, C, T, H, W, t0, nt, Tp, Hp, Wp, (hipStream_t)stream),
                      "cvt_video_pad launch");
}

int cvt_video_unpad(const void* y, void* x, int dtype, int B, int C, int T, int H, int W, int t0, int nt, int Tp,
                    int Hp, int Wp, void* stream) {
    const int st = check_window(y, x, dtype, B, C, T, H, W, t0, nt, Tp, Hp, Wp, Tp);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_video_unpad(y, x, dtype, B, C, T, H, W, t0, nt, Tp, Hp, Wp, (hipStream_t)stream),
                      "cvt_video_unpad launch");
}

int cvt_haar3d_fwd_window(const void* x, int x_dtype, void* y, int y_dtype, int y_layout, int B, int C, int T, int H,
                          int W, int t0, int nt, int Tp, int Hp, int Wp, int temporal_levels, void* stream) {
    const int st = check_haar_window(x, x_dtype, y, y_dtype, y_layout, B, C, T, H, W, t0, nt, Tp, Hp, Wp,
                                     temporal_levels);
    if (st != CVT_OK) return st;
    const cvt::ClipWindow win{T, H, W, t0, nt};
    return hip_status(cvt::launch_haar_fwd(x, x_dtype, y, y_dtype, y_layout, B, C, Tp, Hp, Wp, temporal_levels,
                                           (hipStream_t)stream, &win),
                      "cvt_haar3d_fwd_window launch");
}

int cvt_haar3d_inv_window(const void* y, int y_dtype, int y_layout, void* x, int x_dtype, int B, int C, int T, int H,
                          int W, int t0, int nt, int Tp, int Hp, int Wp, int temporal_levels, void* stream) {
    const int st = check_haar_window(x, x_dtype, y, y_dtype, y_layout, B, C, T, H, W, t0, nt, Tp, Hp, Wp,
                                     temporal_levels);
    if (st != CVT_OK) return st;
    const cvt::ClipWindow win{T, H, W, t0, nt};
    return hip_status(cvt::launch_haar_inv(y, y_dtype, y_layout, x, x_dtype, B, C, Tp, Hp, Wp, temporal_levels,
                                           (hipStream_t)stream, &win),
                      "cvt_haar3d_inv_window launch");
}

int cvt_layernorm3d(const void* x, const float* gamma, const float* beta, void* y, int B, int C, int T, int H, int W,
                    float eps, int swish, void* stream) {
    if (!x || !gamma || !beta || !y) return fail(CVT_E_NULL, "x, gamma, beta and y must not be NULL");
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (C % 8 != 0 || C > 4096) return fail(CVT_E_SHAPE, "C must be a multiple of 8 and at most 4096, got %d", C);
    if (!(eps >= 0.0f)) return fail(CVT_E_SHAPE, "eps must be >= 0");
    if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta))
        return fail(CVT_E_ALIGN, "x, y, gamma and beta must be 16-byte aligned");
    return hip_status(cvt::launch_layernorm(x, gamma, beta, y, (long long)B * T * H * W, C, eps, swish,
                                            (hipStream_t)stream),
                      "cvt_layernorm3d launch");
}

size_t cvt_resblock3d_workspace(int B, int C, int T, int H, int W) {
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0) return 0;
    return cvt::resblock_workspace_bytes(B, C, T, H, W);
}

namespace {
// Arguments of cvt_resblock3d and cvt_resblock3d_packed (packed: the conv weights are the
// 16-byte aligned packed forms).
int check_resblock(const void* x, const cvt_resblock_weights* w, void* y, int B, int C, int T, int H, int W, float eps,
                   void* workspace, size_t workspace_bytes, bool packed) {
    if (!x || !w || !y) return fail(CVT_E_NULL, "x, w and y must not be NULL");
    if (!w->ln1_g || !w->ln1_b || !w->ln2_g || !w->ln2_b || !w->c1_s || !w->c1_t || !w->c2_s || !w->c2_t)
        return fail(CVT_E_NULL, "scales, shifts and conv weights must not be NULL");
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (C < 64 || C % 8 != 0 || !cvt::resblock_supported(C, H, W))
        return fail(CVT_E_SHAPE, "the residual block needs C >= 64, C %% 8 == 0 and 9 frames of a tensor below 2 GiB "
                                 "(C=%d)", C);
    if (!(eps >= 0.0f)) return fail(CVT_E_SHAPE, "eps must be >= 0");
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    for (const float* v : {w->ln1_g, w->ln1_b, w->ln2_g, w->ln2_b})
        if (!aligned16(v)) return fail(CVT_E_ALIGN, "LayerNorm scales and shifts must be 16-byte aligned");
    for (const void* v : {w->c1_s, w->c1_t, w->c2_s, w->c2_t}) {
        if (packed && !aligned16(v)) return fail(CVT_E_ALIGN, "packed weights must be 16-byte aligned");
        if (reinterpret_cast<uintptr_t>(v) & 1u) return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    }
    for (const float* v : {w->c1_bs, w->c1_bt, w->c2_bs, w->c2_bt})
        if (v && (reinterpret_cast<uintptr_t>(v) & 3u)) return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::resblock_workspace_bytes(B, C, T, H, W, packed);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return CVT_OK;
}
}  // namespace

int cvt_resblock3d(const void* x, const cvt_resblock_weights* w, void* y, int B, int C, int T, int H, int W, float eps,
                   void* workspace, size_t workspace_bytes, void* stream) {
    const int st = check_resblock(x, w, y, B, C, T, H, W, eps, workspace, workspace_bytes, false);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_resblock(x, *w, y, B, C, T, H, W, eps, workspace, (hipStream_t)stream),
                      "cvt_resblock3d launch");
}

size_t cvt_resblock3d_packed_workspace(int B, int C, int T, int H, int W) {
    if (B <= 0 || C <= 0 || T <= 0 || H <= 0 || W <= 0) return 0;
    return cvt::resblock_workspace_bytes(B, C, T, H, W, true);
}

int cvt_resblock3d_packed(const void* x, const cvt_resblock_weights* w, void* y, int B, int C, int T, int H, int W,
                          float eps, void* workspace, size_t workspace_bytes, void* stream) {
    const int st = check_resblock(x, w, y, B, C, T, H, W, eps, workspace, workspace_bytes, true);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_resblock(x, *w, y, B, C, T, H, W, eps, workspace, (hipStream_t)stream, true),
                      "cvt_resblock3d_packed launch");
}

size_t cvt_downsample3d_workspace(int B, int Cin, int Cout, int T, int H, int W, int parts) {
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0 || parts < 1 || parts > 3) return 0;
    return cvt::downsample_workspace_bytes(B, Cin, Cout, T, H, W, parts & CVT_CONV_SPATIAL, parts & CVT_CONV_TEMPORAL);
}

namespace {
// Arguments of cvt_downsample3d and cvt_downsample3d_packed (packed: 16-byte aligned packed
// weights, both parts on the row-tiled kernels).
int check_downsample(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                     int B, int Cin, int Cout, int T, int H, int W, void* workspace, size_t workspace_bytes,
                     bool packed) {
    if (!x || !y || (!w_s && !w_t)) return fail(CVT_E_NULL, "x, y and at least one weight must not be NULL");
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (Cin % 8 != 0 || Cout % 8 != 0)
        return fail(CVT_E_SHAPE, "Cin and Cout must be multiples of 8 (got %d, %d)", Cin, Cout);
    if (w_s && (H % 2 || W % 2)) return fail(CVT_E_SHAPE, "spatial downsampling needs even H and W (got %dx%d)", H, W);
    if (w_t && (T - 1) % 2) return fail(CVT_E_SHAPE, "temporal downsampling needs T = 1 + 2k frames (got %d)", T);
    if (packed && (Cout < 64 || !cvt::downsample_packed_supported(Cin, Cout, H, W, w_s != nullptr, w_t != nullptr)))
        return fail(CVT_E_SHAPE, "packed weights run the row-tiled kernels: Cout >= 64, Cin == Cout for the temporal "
                                 "part alone and a tile's rows of the input below 2 GiB (Cin=%d, Cout=%d)", Cin, Cout);
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    if (packed && ((w_s && !aligned16(w_s)) || (w_t && !aligned16(w_t))))
        return fail(CVT_E_ALIGN, "packed weights must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_s) & 1u) || (reinterpret_cast<uintptr_t>(w_t) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::downsample_workspace_bytes(B, Cin, Cout, T, H, W, w_s != nullptr, w_t != nullptr, packed);
    if (need == 0) return CVT_OK;  // packed, one part: no workspace
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return CVT_OK;
}
}  // namespace

int cvt_downsample3d(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                     int B, int Cin, int Cout, int T, int H, int W, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const int st = check_downsample(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, workspace, workspace_bytes, false);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_downsample(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, workspace,
                                             (hipStream_t)stream),
                      "cvt_downsample3d launch");
}

size_t cvt_downsample3d_packed_workspace(int B, int Cin, int Cout, int T, int H, int W, int parts) {
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0 || parts < 1 || parts > 3) return 0;
    return cvt::downsample_workspace_bytes(B, Cin, Cout, T, H, W, parts & CVT_CONV_SPATIAL, parts & CVT_CONV_TEMPORAL,
                                           true);
}

int cvt_downsample3d_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s, const float* b_t,
                            void* y, int B, int Cin, int Cout, int T, int H, int W, void* workspace,
                            size_t workspace_bytes, void* stream) {
    const int st = check_downsample(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W, workspace, workspace_bytes, true);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_downsample(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W, workspace,
                                             (hipStream_t)stream, true),
                      "cvt_downsample3d_packed launch");
}

size_t cvt_upsample3d_workspace(int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time) {
    (void)up_time;
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return 0;
    return cvt::upsample_workspace_bytes(B, Cin, Cout, T, H, W, up_space != 0);
}

namespace {
// Arguments of cvt_upsample3d and cvt_upsample3d_packed (packed: 16-byte aligned packed weights).
int check_upsample(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y, int B,
                   int Cin, int Cout, int T, int H, int W, int up_space, int up_time, void* workspace,
                   size_t workspace_bytes, bool packed) {
    if (!x || !y || !w_s || !w_t) return fail(CVT_E_NULL, "x, y, w_s and w_t must not be NULL");
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    const int f = up_space ? 2 : 1;
    const long long Pout = (long long)B * (up_time ? 2 * T - 1 : T) * f * H * f * W;
    if (Cin % 8 != 0 || Cout % 8 != 0 || Cout < 64 ||
        !cvt::upsample_supported(Cin, Cout, W, (long long)f * H * f * W) ||
        (long long)f * H * f * W * Cout >= (1LL << 30) || Pout * Cout * 2 >= (1LL << 40))
        return fail(CVT_E_SHAPE, "upsampling needs Cin, Cout multiples of 8, Cout >= 64 and 9 frames of the "
                                 "upsampled tensor below 2 GiB (Cin=%d, Cout=%d)", Cin, Cout);
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    if (packed && (!aligned16(w_s) || !aligned16(w_t))) return fail(CVT_E_ALIGN, "packed weights must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_s) & 1u) || (reinterpret_cast<uintptr_t>(w_t) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::upsample_workspace_bytes(B, Cin, Cout, T, H, W, up_space != 0, packed);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return CVT_OK;
}
}  // namespace

int cvt_upsample3d(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y, int B,
                   int Cin, int Cout, int T, int H, int W, int up_space, int up_time, void* workspace,
                   size_t workspace_bytes, void* stream) {
    const int st = check_upsample(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, up_space, up_time, workspace,
                                  workspace_bytes, false);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_upsample(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, up_space != 0,
                                           up_time != 0, workspace, (hipStream_t)stream),
                      "cvt_upsample3d launch");
}

size_t cvt_upsample3d_packed_workspace(int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time) {
    (void)up_time;
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return 0;
    return cvt::upsample_workspace_bytes(B, Cin, Cout, T, H, W, up_space != 0, true);
}

int cvt_upsample3d_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s, const float* b_t,
                          void* y, int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const int st = check_upsample(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W, up_space, up_time, workspace,
                                  workspace_bytes, true);
    if (st != CVT_OK) return st;
    return hip_status(cvt::launch_upsample(x, pw_s, pw_t, b_s, b_t, y, B, Cin, Cout, T, H, W, up_space != 0,
                                           up_time != 0, workspace, (hipStream_t)stream, true),
                      "cvt_upsample3d_packed launch");
}

size_t cvt_causal_conv3d_fact_proj_fsq_workspace(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k,
                                                 int parts) {
    if (B <= 0 || Cin <= 0 || Cout <= 0 || Cp <= 0 || T <= 0 || H <= 0 || W <= 0 || (k != 1 && k != 3)) return 0;
    if (parts < 1 || parts > 3) return 0;
    return cvt::conv_proj_fsq_workspace_bytes(B, Cin, Cout, Cp, T, H, W, k, (parts & CVT_CONV_SPATIAL) != 0,
                                              (parts & CVT_CONV_TEMPORAL) != 0);
}

int cvt_causal_conv3d_fact_proj_fsq(const void* x, const void* w_s, const void* w_t, const float* b_s,
                                    const float* b_t, const void* w_p, const float* b_p, const int32_t* levels, int D,
                                    void* y, int32_t* indices, int B, int Cin, int Cout, int T, int H, int W, int k,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !w_p || !indices) return fail(CVT_E_NULL, "x, w_p and indices must not be NULL");
    if (!w_s && !w_t) return fail(CVT_E_NULL, "at least one of w_s and w_t must be given");
    cvt::FsqParams p;
    const int st = fsq_params(levels, D, &p);
    if (st != CVT_OK) return st;
    const int Cp = D;
    if (B <= 0 || Cin <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (k != 1 && k != 3) return fail(CVT_E_SHAPE, "k must be 1 or 3, got %d", k);
    if (Cout > 4096) return fail(CVT_E_SHAPE, "Cout must be at most 4096, got %d", Cout);
    if (!w_s && Cin != Cout)
        return fail(CVT_E_SHAPE, "a temporal-only call needs Cin == Cout (got %d and %d)", Cin, Cout);
    if (Cin % 8 != 0) return fail(CVT_E_SHAPE, "Cin must be a multiple of 8, got %d", Cin);
    if (Cout % 8 != 0) return fail(CVT_E_SHAPE, "Cout must be a multiple of 8, got %d", Cout);
    if (!aligned16(x) || (y && !aligned16(y)) || !aligned16(indices))
        return fail(CVT_E_ALIGN, "x, y and indices must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_s) & 1u) || (reinterpret_cast<uintptr_t>(w_t) & 1u) ||
        (reinterpret_cast<uintptr_t>(w_p) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)) ||
        (b_p && (reinterpret_cast<uintptr_t>(b_p) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need =
        cvt::conv_proj_fsq_workspace_bytes(B, Cin, Cout, Cp, T, H, W, k, w_s != nullptr, w_t != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(cvt::launch_conv_fact_proj(x, w_s, w_t, b_s, b_t, w_p, b_p, y, B, Cin, Cout, Cp, T, H, W, k,
                                                 workspace, (hipStream_t)stream, indices, &p),
                      "cvt_causal_conv3d_fact_proj_fsq launch");
}

int cvt_fsq_dequantize_proj(const int32_t* indices, const int32_t* levels, int D, const void* w_p, const float* b_p,
                            void* y, int B, int Cout, int T, int H, int W, int32_t* d_invalid_count, void* stream) {
    if (!indices || !w_p || !y) return fail(CVT_E_NULL, "indices, w_p and y must not be NULL");
    cvt::FsqParams p;
    const int st = fsq_params(levels, D, &p);
    if (st != CVT_OK) return st;
    if (B <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (Cout > 4096) return fail(CVT_E_SHAPE, "Cout must be at most 4096, got %d", Cout);
    if (!aligned16(indices) || !aligned16(y)) return fail(CVT_E_ALIGN, "indices and y must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(w_p) & 1u) return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if (b_p && (reinterpret_cast<uintptr_t>(b_p) & 3u)) return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    if (d_invalid_count && (reinterpret_cast<uintptr_t>(d_invalid_count) & 3u))
        return fail(CVT_E_ALIGN, "the invalid counter must be 4-byte aligned");
    return hip_status(cvt::launch_fsq_dequant_proj(indices, p, w_p, b_p, y, (long long)B * T * H * W, Cout,
                                                   d_invalid_count, (hipStream_t)stream),
                      "cvt_fsq_dequantize_proj launch");
}

size_t cvt_haar3d_conv3d_fact_workspace(int B, int Cout, int T, int H, int W, int parts) {
    if (B <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return 0;
    if (parts != CVT_CONV_SPATIAL && parts != (CVT_CONV_SPATIAL | CVT_CONV_TEMPORAL)) return 0;
    return cvt::haar_conv_workspace_bytes(B, Cout, T, H, W, (parts & CVT_CONV_TEMPORAL) != 0);
}

int cvt_haar3d_conv3d_fact(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                           void* y, int B, int Cout, int T, int H, int W, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (!x || !w_s || !y) return fail(CVT_E_NULL, "x, w_s and y must not be NULL");
    if (B <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (T % 4 != 1) return fail(CVT_E_SHAPE, "the clip needs T = 1 + 4k frames, got %d", T);
    if (H % 4 != 0 || W % 4 != 0) return fail(CVT_E_SHAPE, "H and W must be multiples of 4, got %dx%d", H, W);
    if (Cout < 64 || Cout > 4096 || Cout % 8 != 0)
        return fail(CVT_E_SHAPE, "Cout must be a multiple of 8 in 64..4096, got %d", Cout);
    // the fused loads address the clip with 31-bit byte offsets
    if ((long long)B * 3 * T * H * W * 2 >= 0x7fff0000LL) return fail(CVT_E_SHAPE, "the clip must stay below 2 GiB");
    if ((long long)(H / 4) * (W / 4) * (1 + (T - 1) / 4) * B >= (1LL << 31))
        return fail(CVT_E_SHAPE, "too many latent positions");
    if (!aligned16(x) || !aligned16(y)) return fail(CVT_E_ALIGN, "x and y must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_s) & 1u) || (reinterpret_cast<uintptr_t>(w_t) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) || (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::haar_conv_workspace_bytes(B, Cout, T, H, W, w_t != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(cvt::launch_haar_conv(x, w_s, w_t, b_s, b_t, y, B, Cout, T, H, W, workspace, (hipStream_t)stream),
                      "cvt_haar3d_conv3d_fact launch");
}

size_t cvt_fsq_dequantize_conv3d_fact_workspace(int B, int Cmid, int Cout, int T, int H, int W, int parts) {
    if (B <= 0 || Cmid <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return 0;
    if (parts != CVT_CONV_SPATIAL && parts != (CVT_CONV_SPATIAL | CVT_CONV_TEMPORAL)) return 0;
    return cvt::fsq_conv_workspace_bytes(B, Cmid, Cout, T, H, W, (parts & CVT_CONV_TEMPORAL) != 0);
}

int cvt_fsq_dequantize_conv3d_fact(const int32_t* indices, const int32_t* levels, int D, const void* w_lift,
                                   const float* b_lift, const void* w_s, const void* w_t, const float* b_s,
                                   const float* b_t, void* y, int B, int Cmid, int Cout, int T, int H, int W,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (!indices || !w_lift || !w_s || !y) return fail(CVT_E_NULL, "indices, w_lift, w_s and y must not be NULL");
    cvt::FsqParams p;
    const int st = fsq_params(levels, D, &p);
    if (st != CVT_OK) return st;
    if (B <= 0 || Cmid <= 0 || Cout <= 0 || T <= 0 || H <= 0 || W <= 0) return fail(CVT_E_SHAPE, "non-positive size");
    if (Cmid % 32 != 0 || Cmid > 256) return fail(CVT_E_SHAPE, "Cmid must be a multiple of 32 up to 256, got %d", Cmid);
    if (Cout < 64 || Cout > 4096 || Cout % 8 != 0)
        return fail(CVT_E_SHAPE, "Cout must be a multiple of 8 in 64..4096, got %d", Cout);
    if ((long long)B * T * H * W * 4 >= 0x7fff0000LL) return fail(CVT_E_SHAPE, "the indices must stay below 2 GiB");
    if (!aligned16(indices) || !aligned16(y)) return fail(CVT_E_ALIGN, "indices and y must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(w_lift) & 1u) || (reinterpret_cast<uintptr_t>(w_s) & 1u) ||
        (reinterpret_cast<uintptr_t>(w_t) & 1u))
        return fail(CVT_E_ALIGN, "weights must be 2-byte aligned");
    if ((b_lift && (reinterpret_cast<uintptr_t>(b_lift) & 3u)) || (b_s && (reinterpret_cast<uintptr_t>(b_s) & 3u)) ||
        (b_t && (reinterpret_cast<uintptr_t>(b_t) & 3u)))
        return fail(CVT_E_ALIGN, "biases must be 4-byte aligned");
    const size_t need = cvt::fsq_conv_workspace_bytes(B, Cmid, Cout, T, H, W, w_t != nullptr);
    if (!workspace || workspace_bytes < need)
        return fail(CVT_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(CVT_E_ALIGN, "workspace must be 16-byte aligned");
    return hip_status(cvt::launch_fsq_conv(indices, p, w_lift, b_lift, w_s, w_t, b_s, b_t, y, B, Cmid, Cout, T, H, W,
                                           workspace, (hipStream_t)stream),
                      "cvt_fsq_dequantize_conv3d_fact launch");
}

}  // extern "C"
