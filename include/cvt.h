/*
 * cvt.h - C ABI of the causal video tokenizer hot path on AMD MI355X (gfx950).
 *
 * The library computes the encoder front end and quantizer of the Cosmos
 * Tokenizer and their inverses: 2-level Haar wavelet patching with the causal
 * first frame, the factorized causal 3D convolution, FSQ quantization to a
 * mixed-radix index, FSQ dequantization and the inverse Haar transform.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, y, z, w_*, b_*, indices, codes and workspace are DEVICE
 *   pointers (memory from hipMalloc or torch on the same device).  `levels` is
 *   a HOST array read during the call only.  The caller allocates and frees
 *   all memory and owns the stream; the library allocates nothing and keeps no
 *   pointer after it returns.
 * - Every function is asynchronous on `stream` (a hipStream_t; NULL means the
 *   null stream) and returns a cvt_status.  All arguments are validated before
 *   anything is launched: on an error nothing runs and nothing is written.
 *   CVT_E_HIP means a launch failed; cvt_last_error() gives the detail
 *   (thread-local).  No C++ exception crosses this interface.
 * - Dense tensors are contiguous.  A [B, C, T, H, W] tensor is stored either
 *   NCTHW (W fastest) or NTHWC (C fastest, torch's channels_last_3d).
 * - bf16 is IEEE binary32's upper half; conversions to bf16 round to nearest
 *   even.  Device pointers must be 16-byte aligned.
 * - Sizes are int; element counts may exceed 2^31 (the library indexes with
 *   64-bit offsets).
 */
#ifndef CVT_H
#define CVT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CVT_OK = 0,
    CVT_E_NULL = 1,      /* a required pointer is NULL */
    CVT_E_SHAPE = 2,     /* a size is non-positive or violates the operation's shape rule */
    CVT_E_DTYPE = 3,     /* unsupported dtype code */
    CVT_E_LAYOUT = 4,    /* unsupported layout code */
    CVT_E_ALIGN = 5,     /* a device pointer is not 16-byte aligned */
    CVT_E_LEVELS = 6,    /* FSQ levels outside the supported range */
    CVT_E_WORKSPACE = 7, /* workspace missing or smaller than required */
    CVT_E_HIP = 8        /* the HIP runtime reported an error on launch */
} cvt_status;

typedef enum { CVT_F32 = 0, CVT_BF16 = 1 } cvt_dtype;
typedef enum { CVT_NCTHW = 0, CVT_NTHWC = 1 } cvt_layout;

/* Version of this interface (incremented on any signature change). */
int cvt_abi_version(void);
/* Static string naming a status code. */
const char* cvt_status_string(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* cvt_last_error(void);

/*
 * Forward Haar patcher with the causal first frame.
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南" (a guide to the tokenizer
 * README), section 7.1 (Haar wavelet patching) and sections 6.1 / 7.3 (first
 * latent frame aligned with frame 0, T' = 1 + (T-1)/4); the
 * Cosmos-Tokenize1-CV8x8x8-720p model card, "Model Architecture" (the encoder
 * starts with a 2-level Haar transform, 4x in T, H and W).
 *
 * x: [B, C, T, H, W] NCTHW, dtype x_dtype (CVT_F32 or CVT_BF16).
 * temporal_levels = 2 (video): T = 1 + 4k; the sequence is extended by three
 *   leading copies of frame 0 and two orthonormal Haar levels are applied along
 *   t, h and w.  y: [B, 64C, T', H/4, W/4] with T' = 1 + (T-1)/4.
 * temporal_levels = 0 (image patcher, per frame): two levels along h and w.
 *   y: [B, 16C, T, H/4, W/4].
 * temporal_levels = 3 (continuation chunk of a stream): T = 4k frames, no
 *   leading copies; latent frame j is made of frames 4j .. 4j+3, so encoding a
 *   clip's frames 0 .. 4a as one temporal_levels = 2 call and the following 4k
 *   frames as a temporal_levels = 3 call gives exactly the latent frames of one
 *   call over the whole clip (the causal design: a frame depends only on itself
 *   and earlier frames).  y: [B, 64C, T/4, H/4, W/4].
 * Output channel = s2*G*C + s1*C + c with G = 8 (3D) or 4 (2D), where s1, s2
 * are the level-1 and level-2 subbands, s = 4*b_t + 2*b_h + b_w (2D:
 * 2*b_h + b_w), b = 0 for the low-pass (e+o)/sqrt(2) and 1 for the high-pass
 * (e-o)/sqrt(2), e being the earlier / upper / left sample of a pair.
 * y is stored in y_layout (NTHWC is the layout the convolution consumes) with
 * dtype y_dtype.  Arithmetic is float32.
 * Errors: CVT_E_SHAPE if H or W is not a multiple of 4, T is not 1 + 4k with
 * temporal_levels = 2 or 4k with temporal_levels = 3, or temporal_levels is not
 * 0, 2 or 3.
 */
int cvt_haar3d_fwd(const void* x, int x_dtype, void* y, int y_dtype, int y_layout,
                   int B, int C, int T, int H, int W, int temporal_levels, void* stream);

/*
 * Inverse Haar patcher (the decoder's last layer).
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 7.1 (the inverse
 * wavelet transform restores the pixels); Cosmos-Tokenize1-CV8x8x8-720p model
 * card, "Model Architecture" (the decoder ends with an inverse wavelet
 * transform).
 *
 * y: coefficients as produced by cvt_haar3d_fwd, layout y_layout, dtype
 * y_dtype.  x: output [B, C, T, H, W] NCTHW, dtype x_dtype, where T, H, W are
 * the PIXEL sizes (T = 4T' - 3 with temporal_levels = 2, the three leading
 * padded frames being dropped; T = 4T' for a continuation chunk,
 * temporal_levels = 3; T = T' with temporal_levels = 0).
 * Errors: as cvt_haar3d_fwd.
 */
int cvt_haar3d_inv(const void* y, int y_dtype, int y_layout, void* x, int x_dtype,
                   int B, int C, int T, int H, int W, int temporal_levels, void* stream);

/*
 * Factorized causal 3D convolution: a 1 x k x k spatial convolution
 * (Cin -> Cout, zero padding (k-1)/2 in H and W, cross-correlation) followed by
 * a k x 1 x 1 temporal convolution (Cout -> Cout) with k-1 zero frames of left
 * padding, so output frame t depends on frames t-k+1 .. t only.
 *
 * Defined by: "Cosmos World Foundation Model Platform for Physical AI
 * (Cosmos-Predict1)" summary, section "1) Cosmos Tokenizer" (1 x k x k then
 * k x 1 x 1 with left padding k-1 for causality); model card "Model
 * Architecture" (causal temporal convolution).
 *
 * x:   bf16 NTHWC [B, Cin, T, H, W]; Cin a multiple of 8 (or Cin <= 16
 *      for a spatial-only call with k = 1).
 * w_s: bf16 [Cout, Cin, 1, k, k] (torch's Conv3d weight order), or NULL for
 *      the temporal part alone (then Cin must equal Cout).
 * w_t: bf16 [Cout, Cout, k, 1, 1], or NULL for the spatial part alone
 *      (with k = 1 and w_t = NULL the call is a 1x1x1 projection).
 *      At least one of w_s and w_t must be given.
 * b_s, b_t: float32 [Cout] biases or NULL.
 * y:   bf16 NTHWC [B, Cout, T, H, W]; must not overlap x, the weights or the
 *      workspace (a tile reads input rows and frames that the outputs of other
 *      tiles would overwrite).
 * k:   1 or 3.
 * Accumulation is float32; the spatial result is stored as bf16 in the
 * workspace before the temporal convolution reads it.
 * workspace: device scratch of at least cvt_causal_conv3d_fact_workspace()
 * bytes (packed weights and, when both parts run, the intermediate), owned by
 * the caller; `parts` there is CVT_CONV_SPATIAL | CVT_CONV_TEMPORAL for the
 * parts the call will run (0 is returned for invalid arguments).
 * Errors: CVT_E_SHAPE for k not 1 or 3, Cin or Cout out of range (Cin must
 * be a multiple of 8, or at most 16 with k = 1; 1 <= Cout <= 4096);
 * CVT_E_WORKSPACE when workspace_bytes is too small.
 */
enum { CVT_CONV_SPATIAL = 1, CVT_CONV_TEMPORAL = 2 };
size_t cvt_causal_conv3d_fact_workspace(int B, int Cin, int Cout, int T, int H, int W, int k, int parts);
int cvt_causal_conv3d_fact(const void* x, const void* w_s, const void* w_t,
                           const float* b_s, const float* b_t, void* y,
                           int B, int Cin, int Cout, int T, int H, int W, int k,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * cvt_causal_conv3d_fact for callers that cannot allocate (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): the same operation,
 * kernels and result bit for bit, with the workspace replaced by scratch memory
 * the library preallocates, a device array of CVT_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing and calls no allocating routine; the caller passes inputs
 * and outputs only.
 *
 * Arguments and errors: as cvt_causal_conv3d_fact without the workspace;
 * CVT_E_WORKSPACE (nothing launched) when the call would need more scratch than
 * CVT_NOALLOC_SCRATCH_BYTES, i.e. when cvt_causal_conv3d_fact_workspace() for
 * the same arguments exceeds it (the packed weights, plus the bf16 intermediate
 * of B*T*H*W*Cout*2 bytes when both parts run: about 125,000 positions at
 * 256 channels; a single part needs only its packed weights).
 * Every call on one GPU uses that GPU's single copy of the scratch: calls that
 * overlap on one GPU (two streams, two host threads) race and must be ordered
 * by the caller.  The first call on a device looks up the scratch's address
 * (hipGetSymbolAddress) on the calling thread's current device, which must be
 * the device of the tensors and the stream.
 */
#define CVT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int cvt_causal_conv3d_fact_noalloc(const void* x, const void* w_s, const void* w_t,
                                   const float* b_s, const float* b_t, void* y,
                                   int B, int Cin, int Cout, int T, int H, int W, int k,
                                   void* stream);

/*
 * Conv weights packed once, for callers whose weights stay fixed across calls
 * (inference): the same operations as cvt_causal_conv3d_fact (k = 3) and
 * cvt_causal_conv3d_fact_proj, without the per-call weight repack.  Source:
 * as cvt_causal_conv3d_fact ("Cosmos World Foundation Model Platform for
 * Physical AI (Cosmos-Predict1)", section "1) Cosmos Tokenizer").
 *
 * cvt_conv_weights_packed_bytes(Cout, Cin, taps): bytes of the packed form of a
 *      bf16 weight tensor [Cout, Cin, taps] in torch order: taps = 9 (1x3x3
 *      spatial), 3 (3x1x1 temporal) or 1 (1x1 projection); 0 for invalid
 *      arguments.
 * cvt_conv_weights_pack: writes that packed form of w into `packed` (device,
 *      16-byte aligned, owned by the caller, at least that many bytes) on the
 *      stream: the order in which the row-tiled convolution kernels read their
 *      weights (1 KB fragments of 32 output x 16 input channels, zeros past
 *      Cout and Cin).  The projection of the _proj call is packed with
 *      Cout = Cp, Cin = the conv's Cout, taps = 1.
 *      Errors: CVT_E_NULL, CVT_E_SHAPE (Cout or Cin outside 1..4096, taps not
 *      1, 3 or 9), CVT_E_ALIGN (w not 2-byte, packed not 16-byte aligned).
 * cvt_causal_conv3d_fact_packed: x, b_s, b_t, y, sizes as
 *      cvt_causal_conv3d_fact with k = 3; pw_s, pw_t: the packed spatial
 *      (taps 9) and temporal (taps 3) weights, either NULL as there.
 *      workspace: cvt_causal_conv3d_fact_packed_workspace() bytes (the bf16
 *      intermediate when both parts run; 0, and workspace may be NULL, for one
 *      part).
 * cvt_causal_conv3d_fact_proj_packed: as cvt_causal_conv3d_fact_proj with
 *      k = 3 and packed weights; the temporal part (pw_t) and the projection
 *      (pw_p, Cp channels) are required, the projection runs in the temporal
 *      convolution's epilogue.  workspace: the spatial part's bf16 output when
 *      pw_s is given (cvt_causal_conv3d_fact_proj_packed_workspace, parts =
 *      CVT_CONV_TEMPORAL or CVT_CONV_SPATIAL | CVT_CONV_TEMPORAL), else none.
 * The outputs equal those of the unpacked calls bit for bit.
 * Errors: CVT_E_NULL (x, y; both pw_s and pw_t NULL; for _proj pw_t or pw_p);
 *      CVT_E_SHAPE for Cin or Cout not a multiple of 8, Cout < 64 or above
 *      4096, a temporal-only call with Cin != Cout, shapes the row-tiled
 *      kernels do not take (10 image rows or 9 frames of the input of 2 GiB
 *      or more), and for _proj Cout > 256 or Cp outside 1..16; CVT_E_ALIGN
 *      unless x, y, the packed weights and the workspace are 16-byte and the
 *      biases 4-byte aligned; CVT_E_WORKSPACE when the workspace is too small.
 */
size_t cvt_conv_weights_packed_bytes(int Cout, int Cin, int taps);
int cvt_conv_weights_pack(const void* w, void* packed, int Cout, int Cin, int taps, void* stream);
size_t cvt_causal_conv3d_fact_packed_workspace(int B, int Cout, int T, int H, int W, int parts);
int cvt_causal_conv3d_fact_packed(const void* x, const void* pw_s, const void* pw_t,
                                  const float* b_s, const float* b_t, void* y,
                                  int B, int Cin, int Cout, int T, int H, int W,
                                  void* workspace, size_t workspace_bytes, void* stream);
size_t cvt_causal_conv3d_fact_proj_packed_workspace(int B, int Cout, int T, int H, int W, int parts);
int cvt_causal_conv3d_fact_proj_packed(const void* x, const void* pw_s, const void* pw_t,
                                       const float* b_s, const float* b_t, const void* pw_p,
                                       const float* b_p, void* y, int B, int Cin, int Cout, int Cp,
                                       int T, int H, int W, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Factorized causal convolution (as cvt_causal_conv3d_fact) followed by a
 * 1x1x1 projection to Cp channels, without writing the Cout-channel result:
 *   y = bf16( w_p . bf16(conv(x)) + b_p ),
 * i.e. the same two roundings as calling cvt_causal_conv3d_fact and then the
 * k = 1 projection on its bf16 output; only the float32 summation order of the
 * projection differs.
 *
 * Defined by: "Cosmos World Foundation Model Platform for Physical AI
 * (Cosmos-Predict1)" summary, section "1) Cosmos Tokenizer" (the factorized
 * causal convolution) and the model card's "Input/Output Specifications"
 * (latent width: 16 continuous channels, 6 FSQ channels) for the projection
 * to the latent.
 *
 * x, w_s, w_t, b_s, b_t, B, Cin, Cout, T, H, W, k: as cvt_causal_conv3d_fact,
 *      with Cin and Cout multiples of 8.
 * w_p: bf16 [Cp, Cout, 1, 1, 1] (torch's Conv3d weight order); b_p: float32
 *      [Cp] or NULL.
 * y:   bf16 NTHWC [B, Cp, T, H, W].
 * The projection runs inside the temporal convolution's epilogue when the
 * temporal part is given, k = 3, Cout <= 256 and Cp <= 16; otherwise the
 * convolution output is materialised in the workspace and projected by a
 * second pass (same result).
 * workspace: device scratch of at least cvt_causal_conv3d_fact_proj_workspace()
 * bytes, owned by the caller (`parts` as for cvt_causal_conv3d_fact_workspace;
 * 0 is returned for invalid arguments).
 * Errors: as cvt_causal_conv3d_fact; CVT_E_NULL also when w_p is NULL;
 * CVT_E_SHAPE also for Cp outside 1..4096 or Cin or Cout not a multiple of 8.
 */
size_t cvt_causal_conv3d_fact_proj_workspace(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k, int parts);
int cvt_causal_conv3d_fact_proj(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                                const void* w_p, const float* b_p, void* y, int B, int Cin, int Cout, int Cp,
                                int T, int H, int W, int k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The factorized conv with the 1x1 projection to the D-dim latent AND its FSQ
 * quantization (cvt_fsq_quantize of the bf16 latent) in one pass: where the
 * projection runs in the temporal conv's epilogue (temporal part present,
 * k = 3, Cout <= 256, D <= 8) the indices are computed there and the latent
 * need not be written; otherwise the latent goes through the FSQ kernel.
 * Either way indices equal cvt_fsq_quantize of cvt_causal_conv3d_fact_proj's
 * output bit for bit.
 *
 * Defined by: the Cosmos-Predict1 summary, section "1) Cosmos Tokenizer" (the
 * discrete tokenizer quantizes a 6-dim latent with FSQ levels (8,8,8,5,5,5))
 * and "NVIDIA Cosmos Tokenizer 完全指南", section 7.2 (FSQ).
 *
 * Arguments as cvt_causal_conv3d_fact_proj with Cp = D, plus levels (host
 * int32[D]) and indices (int32 [B, T, H, W], 16-byte aligned); y (the bf16
 * NTHWC latent [B, D, T, H, W]) may be NULL.  workspace:
 * cvt_causal_conv3d_fact_proj_fsq_workspace(..., Cp = D, ...) bytes.
 * Errors: as cvt_causal_conv3d_fact_proj and cvt_fsq_quantize.
 */
size_t cvt_causal_conv3d_fact_proj_fsq_workspace(int B, int Cin, int Cout, int Cp, int T, int H, int W, int k,
                                                 int parts);
int cvt_causal_conv3d_fact_proj_fsq(const void* x, const void* w_s, const void* w_t, const float* b_s,
                                    const float* b_t, const void* w_p, const float* b_p, const int32_t* levels, int D,
                                    void* y, int32_t* indices, int B, int Cin, int Cout, int T, int H, int W, int k,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal temporal convolution (k = 3) of one chunk of a stream, optionally followed
 * by the fused 1x1x1 projection:
 *   y[t] = sum_j w_t[:, :, j] . x[t + j - 2] (+ b_t),   t = 0 .. T-1,
 * where x[-2] and x[-1] are the two frames of `hist` (the last two frames of the
 * previous chunk's input), or zeros when hist is NULL (the start of a stream: the
 * causal left padding of cvt_causal_conv3d_fact).  Running a clip chunk by chunk
 * this way gives bit for bit the result of one call over the whole clip, so clips
 * of any length can be encoded with memory bounded by the chunk size.
 *
 * Defined by: "Cosmos World Foundation Model Platform for Physical AI
 * (Cosmos-Predict1)" summary, section "1) Cosmos Tokenizer" (the temporal
 * convolution is causal with k - 1 frames of left padding) and the guide's
 * section 6.3 (videos of any length).
 *
 * x: bf16 NTHWC [B, C, T, H, W]; hist: NULL or bf16 NTHWC [B, C, 2, H, W] (with
 *    B = 1 it may point into the previous chunk's buffer at its frame T_prev - 2);
 * w_t: bf16 [C, C, 3, 1, 1]; b_t: float32 [C] or NULL;
 * w_p: NULL (y = the convolution, bf16 NTHWC [B, C, T, H, W]) or bf16
 *    [Cp, C, 1, 1, 1] with C <= 256 and 1 <= Cp <= 16 (y = the projection,
 *    bf16 NTHWC [B, Cp, T, H, W], rounded as cvt_causal_conv3d_fact_proj);
 *    b_p: float32 [Cp] or NULL.
 * workspace: at least cvt_causal_conv3d_temporal_stream_workspace(C, Cp) bytes
 *    (Cp = 0 without projection); owned by the caller.
 * Errors: CVT_E_NULL for a NULL x, w_t or y; CVT_E_SHAPE for a non-positive
 * size, C < 64, C not a multiple of 8, a projection outside the limits above or
 * 9 frames of the input (9*H*W*C*2 bytes) of 2 GiB or more (the input itself
 * may have any size); CVT_E_ALIGN unless x, hist and y are 16-byte
 * aligned; CVT_E_WORKSPACE when the workspace is too small.
 */
size_t cvt_causal_conv3d_temporal_stream_workspace(int C, int Cp);
int cvt_causal_conv3d_temporal_stream(const void* x, const void* hist, const void* w_t, const float* b_t,
                                      const void* w_p, const float* b_p, void* y, int B, int C, int Cp, int T,
                                      int H, int W, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Factorized causal self-attention core, one axis per call:
 *   out = softmax(q k^T / sqrt(d) [+ causal mask]) v   per head,
 * with the C channels split into `heads` heads of d = C / heads consecutive
 * channels (head g = channels g*d .. g*d + d - 1).
 *   axis = CVT_ATTN_SPATIAL: the tokens are the H*W positions of one frame of
 *          one clip, every position attending to every position of the frame.
 *   axis = CVT_ATTN_TEMPORAL_CAUSAL: the tokens are the T frames of one position
 *          of one clip; frame t attends to frames s <= t only.
 *
 * Defined by: "Cosmos World Foundation Model Platform for Physical AI
 * (Cosmos-Predict1)" summary, section "1) Cosmos Tokenizer" (space-time
 * factorized causal self-attention next to the factorized convolution) and the
 * model card's "Model Architecture" (causal temporal attention keeps the frame
 * order).  The pages give no formula, head count or width: scaled dot-product
 * attention with consecutive-channel heads is the reading taken.
 *
 * q, k, v: bf16 NTHWC (torch channels_last_3d) [B, C, T, H, W], produced by the
 *      caller (e.g. 1x1x1 convolutions of a feature map).
 * out: bf16 NTHWC [B, C, T, H, W]; must not overlap q, k or v.
 * Scores, softmax and accumulation are float32; the probabilities are rounded
 * to bf16 for the P v product; out is rounded to bf16 once.
 * Errors: CVT_E_NULL for a NULL tensor; CVT_E_ALIGN unless all four are
 * 16-byte aligned; CVT_E_LAYOUT for an unknown axis; CVT_E_SHAPE for a
 * non-positive size, heads not dividing C, C not a multiple of 8 or above
 * 4096, a head dim d = C / heads that is not a multiple of 8 or above 256, or
 * a frame of H * W * C elements of 2^30 or more.
 * Kernels: spatial head dims 32, 64 and 128 run tiled flash attention on the
 * matrix cores; temporal head dim 64 with T <= 32 one MFMA block per
 * sequence, head dims 32 and 64 with T * C <= 16384 an LDS-staged kernel;
 * every other shape (any head dim up to 256, any T) a one-thread-per-query
 * kernel reading global memory, with the same numerics except that its
 * probabilities stay float32.
 */
enum { CVT_ATTN_SPATIAL = 0, CVT_ATTN_TEMPORAL_CAUSAL = 1 };
int cvt_attention3d(const void* q, const void* k, const void* v, void* out, int B, int C, int T, int H, int W,
                    int heads, int axis, void* stream);

/*
 * FSQ quantization: per position, D latent values -> one int32 index.
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 7.2 (each channel
 * bounded with tanh and rounded to its own number of levels; the index is the
 * mixed-radix number of the digits; codebook size = product of levels =
 * 64000 for (8,8,8,5,5,5)) and section 6.2 (indices [B,T',H',W'], codes
 * [B,6,T',H',W']); the bound is the FSQ method's
 * tanh(z + atanh(o/h)) * h - o with h = (L-1)(1+1e-3)/2, o = 1/2 for even L
 * else 0, rounded half to even; digit d = q + floor(L/2); index =
 * sum_i d_i * prod_{j<i} L_j (channel 0 least significant).
 *
 * z: [B, D, T, H, W] in z_layout, dtype z_dtype.  indices: int32 [B, T, H, W].
 * codes: NULL or an output like z receiving the quantized codes
 * q / floor(L/2) in [-1, 1].  levels: host int32[D].
 * The digit is decided exactly: z is compared with the breakpoints where the
 * bound crosses a half-integer, computed in double precision on the host.
 * A NaN in any channel gives index -1 (and NaN codes); +-inf saturate.
 * Errors: CVT_E_LEVELS unless 1 <= D <= 8, 2 <= L_i <= 16 and the product
 * of the levels is below 2^31.
 */
int cvt_fsq_quantize(const void* z, int z_dtype, int z_layout, int32_t* indices, void* codes,
                     const int32_t* levels, int D, int B, int T, int H, int W, void* stream);

/*
 * FSQ dequantization: index -> digits d_i = floor(idx / beta_i) mod L_i ->
 * codes (d_i - floor(L_i/2)) / floor(L_i/2).
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 7.2
 * (indices_to_codes restores the codes from the index).
 *
 * indices: int32 [B, T, H, W].  codes: output [B, D, T, H, W] in c_layout,
 * dtype c_dtype.  levels: host int32[D].
 * An index outside [0, prod L) is invalid: its codes are NaN and, when
 * d_invalid_count is not NULL, the number of invalid indices is ADDED to the
 * int32 device counter it points to (the caller zeroes it beforehand).
 * Errors: as cvt_fsq_quantize.
 */
int cvt_fsq_dequantize(const int32_t* indices, void* codes, int c_dtype, int c_layout,
                       const int32_t* levels, int D, int B, int T, int H, int W,
                       int32_t* d_invalid_count, void* stream);

/*
 * Sliding windows over a video of any length and size.
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 6.3 (videos of any
 * length are worked through in windows of temporal_window frames, 17 in the
 * guide; each window is padded to the sizes the network accepts, with zeros in
 * space and by reflection at the edge in time, and cropped back after
 * reconstruction) and sections 6.1 / 7.3 (a causal clip holds 1 + k*f frames
 * for a temporal compression f).
 *
 * cvt_video_window: host arithmetic, no device work.  The windows are
 * consecutive: window i holds frames t0 = i*window .. t0 + nt - 1 with
 * nt = min(window, T - t0); there are n_windows = ceil(T / window).  Its padded
 * size is Tp = the smallest 1 + k*t_align >= nt, Hp and Wp = the smallest
 * multiples of s_align >= H and >= W.  Each output pointer may be NULL.
 * Errors: CVT_E_SHAPE for a non-positive argument, index outside
 * [0, n_windows) or a padded size above INT_MAX.
 */
int cvt_video_window(int T, int H, int W, int window, int t_align, int s_align, int index, int* n_windows,
                     int* t0, int* nt, int* Tp, int* Hp, int* Wp);

/*
 * Pad window (t0, nt) of a clip: x [B, C, T, H, W] NCTHW -> y [B, C, Tp, Hp, Wp]
 * NCTHW, both of dtype (CVT_F32 or CVT_BF16), a bit-exact copy:
 *   y[b,c,t,h,w] = x[b,c,t0 + r(t),h,w] for h < H and w < W, else 0,
 * with r(t) = t for t < nt, continued past the last frame by the mirror about
 * it that does not repeat it (nt-2, nt-3, ...), bouncing between the window's
 * two ends when the pad is longer than the window; r = 0 when nt = 1.
 * Padding goes after the content, so the crop keeps indices.
 * Any Tp >= nt, Hp >= H, Wp >= W are accepted (cvt_video_window gives the
 * aligned ones).  y must not overlap x.
 * Errors: CVT_E_NULL, CVT_E_DTYPE; CVT_E_SHAPE for a non-positive size, a
 * window outside the clip, a padded size below the window's, a plane of
 * Hp*Wp elements at or above 2^30 or B*C*Tp at or above 2^31; CVT_E_ALIGN
 * unless x and y are 16-byte aligned.
 */
int cvt_video_pad(const void* x, void* y, int dtype, int B, int C, int T, int H, int W, int t0, int nt, int Tp,
                  int Hp, int Wp, void* stream);

/*
 * Crop a processed padded window y [B, C, Tp, Hp, Wp] NCTHW back to its nt
 * frames and H x W pixels and write it at frames t0 .. t0 + nt - 1 of the clip
 * x [B, C, T, H, W] NCTHW (other frames of x are left untouched), dtype as
 * cvt_video_pad:  x[b,c,t0+t,h,w] = y[b,c,t,h,w].
 * Errors: as cvt_video_pad.
 */
int cvt_video_unpad(const void* y, void* x, int dtype, int B, int C, int T, int H, int W, int t0, int nt, int Tp,
                    int Hp, int Wp, void* stream);

/*
 * Haar patcher of one sliding window, with the window's padding and cropping
 * done inside the transform's own loads and stores.
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 6.3 (windows of a
 * video of any length, padded, reconstructed and cropped back) and section 7.1
 * (Haar wavelet patching), as for cvt_video_pad and cvt_haar3d_fwd.
 *
 * cvt_haar3d_fwd_window gives, bit for bit, what cvt_video_pad of window
 * (t0, nt) to Tp x Hp x Wp followed by cvt_haar3d_fwd of that padded window
 * gives, without writing the padded window: x is the clip [B, C, T, H, W]
 * NCTHW (dtype x_dtype), y the coefficients of the padded window in y_layout /
 * y_dtype, shaped as cvt_haar3d_fwd shapes them for a Tp x Hp x Wp input.
 * cvt_haar3d_inv_window gives what cvt_haar3d_inv of y to a Tp x Hp x Wp
 * window followed by cvt_video_unpad into frames t0 .. t0+nt-1 of the clip x
 * gives: only the window's nt frames, H rows and W columns of x are written.
 * temporal_levels: 2 (Tp = 1 + 4k, each window starts with its own causal
 * first frame) or 0 (per-frame); a continuation chunk (3) is not a window.
 * Hp and Wp are multiples of 4; the clip's H and W may be any size (a width
 * that is not a multiple of 4 takes an element-by-element path).
 * Errors: those of cvt_video_pad / cvt_video_unpad for the window and of
 * cvt_haar3d_fwd / cvt_haar3d_inv for the padded sizes; CVT_E_SHAPE for
 * temporal_levels 3.
 */
int cvt_haar3d_fwd_window(const void* x, int x_dtype, void* y, int y_dtype, int y_layout, int B, int C, int T,
                          int H, int W, int t0, int nt, int Tp, int Hp, int Wp, int temporal_levels, void* stream);
int cvt_haar3d_inv_window(const void* y, int y_dtype, int y_layout, void* x, int x_dtype, int B, int C, int T,
                          int H, int W, int t0, int nt, int Tp, int Hp, int Wp, int temporal_levels, void* stream);

/*
 * Encoder and decoder blocks.
 *
 * Defined by: "Cosmos World Foundation Model Platform for Physical AI
 * (Cosmos-Predict1)" summary, section "1) Cosmos Tokenizer" (after the Haar
 * transform the encoder is residual blocks and downsampling blocks built from
 * the factorized causal convolution, with Swish activations and LayerNorm
 * rather than GroupNorm; the video compression factors are 4x8x8, 8x8x8 and
 * 8x16x16) and the CV8x8x8-720p model card, "Model Architecture" (the decoder
 * mirrors the encoder).  The pages give no block diagram; the readings taken:
 * LayerNorm normalizes the C channels of each position (biased variance, eps
 * inside the square root) and applies a per-channel scale and shift;
 * Swish(x) = x * sigmoid(x); the residual block is the pre-activation form;
 * downsampling is the factorized conv at stride 2; upsampling is
 * nearest-neighbour repetition followed by the factorized conv.
 *
 * All tensors are bf16 NTHWC [B, C, T, H, W] (torch channels_last_3d), 16-byte
 * aligned; scales, shifts and biases float32 (scales and shifts 16-byte
 * aligned); conv weights bf16 in torch's [Cout, Cin, kT, kH, kW] order.
 * Outputs must not overlap inputs.  Arithmetic is float32 with bf16
 * intermediates between the steps listed.
 */

/*
 * y = LN(x) * gamma + beta over the C channels of each position, then Swish if
 * swish != 0.  y may equal x.  Errors: CVT_E_NULL; CVT_E_SHAPE for a
 * non-positive size, C not a multiple of 8 or above 4096; CVT_E_ALIGN.
 */
int cvt_layernorm3d(const void* x, const float* gamma, const float* beta, void* y, int B, int C, int T, int H,
                    int W, float eps, int swish, void* stream);

/* Weights of one residual block over C channels. */
typedef struct cvt_resblock_weights {
    const float* ln1_g; /* [C] scale and shift of the first LayerNorm */
    const float* ln1_b;
    const void* c1_s;   /* bf16 [C, C, 1, 3, 3]: first factorized conv, spatial part */
    const void* c1_t;   /* bf16 [C, C, 3, 1, 1]: its causal temporal part */
    const float* c1_bs; /* [C] or NULL */
    const float* c1_bt; /* [C] or NULL */
    const float* ln2_g; /* second LayerNorm */
    const float* ln2_b;
    const void* c2_s;   /* second factorized conv */
    const void* c2_t;
    const float* c2_bs;
    const float* c2_bt;
} cvt_resblock_weights;

/*
 * Residual block: y = x + conv2(swish(LN2(conv1(swish(LN1(x)))))), conv = the
 * factorized causal conv C -> C with k = 3 (1x3x3 zero padding 1, then 3x1x1
 * with two zero frames in front).  The second LayerNorm and Swish run in the
 * first conv's epilogue for C <= 256, the residual add in the second conv's
 * epilogue (one rounding).  y may be x (in place): the epilogue reads each
 * residual element before the same wave overwrites it.
 * workspace: cvt_resblock3d_workspace(B, C, T, H, W) bytes, caller-owned.
 * Errors: CVT_E_NULL for a NULL tensor, weight or scale/shift; CVT_E_SHAPE for
 * a non-positive size, C < 64, C not a multiple of 8 or 9 frames of the
 * tensor (9*H*W*C*2 bytes) of 2 GiB or more (the tensor itself may have any
 * size); CVT_E_ALIGN; CVT_E_WORKSPACE.
 */
size_t cvt_resblock3d_workspace(int B, int C, int T, int H, int W);
int cvt_resblock3d(const void* x, const cvt_resblock_weights* w, void* y, int B, int C, int T, int H, int W,
                   float eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The residual block on weights packed once, for callers whose weights stay
 * fixed (inference): the same operation and kernels as cvt_resblock3d, bit for
 * bit the same y, without its four per-call weight repacks.  Source: as
 * cvt_resblock3d ("Cosmos World Foundation Model Platform for Physical AI
 * (Cosmos-Predict1)", section "1) Cosmos Tokenizer").  In w, c1_s and c2_s hold
 * the packed forms of the [C, C, 1, 3, 3] weights (cvt_conv_weights_pack with
 * Cout = Cin = C, taps = 9) and c1_t and c2_t those of the [C, C, 3, 1, 1]
 * weights (taps = 3), each 16-byte aligned, device, caller-owned; the other
 * fields are as for cvt_resblock3d.
 * workspace: cvt_resblock3d_packed_workspace(B, C, T, H, W) bytes (the two
 * intermediate tensors only), caller-owned.
 * Errors: as cvt_resblock3d; CVT_E_ALIGN also for packed weights that are not
 * 16-byte aligned.
 */
size_t cvt_resblock3d_packed_workspace(int B, int C, int T, int H, int W);
int cvt_resblock3d_packed(const void* x, const cvt_resblock_weights* w, void* y, int B, int C, int T, int H, int W,
                          float eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Downsampling block: the 1x3x3 conv Cin -> Cout at stride 2 in H and W (zero
 * padding 1: H, W -> H/2, W/2), then the causal 3x1x1 conv at stride 2 in time
 * (two zero frames in front: T = 1 + 2k -> 1 + k, output frame 0 from frame 0
 * alone, output frame j from frames 2j-2 .. 2j).  Either weight may be NULL to
 * skip that part (w_t is then [Cout, Cin, 3, 1, 1] when w_s is NULL).
 * x: [B, Cin, T, H, W]; y: [B, Cout, T', H', W'].
 * parts for the workspace query: CVT_CONV_SPATIAL | CVT_CONV_TEMPORAL.
 * Errors: CVT_E_NULL (both weights NULL); CVT_E_SHAPE for a non-positive
 * size, Cin not a multiple of 8, odd H or W with w_s, T not 1 + 2k with w_t;
 * CVT_E_ALIGN; CVT_E_WORKSPACE.
 */
size_t cvt_downsample3d_workspace(int B, int Cin, int Cout, int T, int H, int W, int parts);
int cvt_downsample3d(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                     int B, int Cin, int Cout, int T, int H, int W, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * The downsampling block on weights packed once (fixed weights): pw_s and pw_t
 * are the packed forms (cvt_conv_weights_pack, taps 9 and 3) of w_s and w_t,
 * 16-byte aligned, either NULL to skip that part; the same kernels and y bit
 * for bit as cvt_downsample3d, without its per-call repacks.  Source: as
 * cvt_downsample3d.  workspace: cvt_downsample3d_packed_workspace bytes (the
 * intermediate of a two-part call; 0 for one part, workspace may then be NULL).
 * Errors: as cvt_downsample3d; CVT_E_SHAPE also where a part would not run on
 * the row-tiled kernels (Cout < 64, a temporal part alone with Cin != Cout,
 * or 10 image rows / 9 frames of the input of 2 GiB or more); CVT_E_ALIGN also
 * for packed weights that are not 16-byte aligned.
 */
size_t cvt_downsample3d_packed_workspace(int B, int Cin, int Cout, int T, int H, int W, int parts);
int cvt_downsample3d_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s, const float* b_t,
                            void* y, int B, int Cin, int Cout, int T, int H, int W, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Upsampling block (the decoder's mirror of downsampling): nearest-neighbour
 * repetition x2 in H and W (up_space) and/or causal repetition in time
 * (up_time: frame 0 once, every later frame twice, T -> 2T - 1), then the
 * factorized conv Cin -> Cout (w_s [Cout, Cin, 1, 3, 3], w_t [Cout, Cout, 3,
 * 1, 1], both required).  The repetition happens inside the conv's loads.
 * x: [B, Cin, T, H, W]; y: [B, Cout, T', 2H or H, 2W or W].
 * Errors: CVT_E_NULL; CVT_E_SHAPE for a non-positive size, Cin or Cout not a
 * multiple of 8, Cout < 64 or 9 frames of the upsampled tensor of 2 GiB or
 * more (the tensors themselves may have any size); CVT_E_ALIGN;
 * CVT_E_WORKSPACE.
 */
size_t cvt_upsample3d_workspace(int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time);
int cvt_upsample3d(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t, void* y,
                   int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * The upsampling block on weights packed once (fixed weights): pw_s and pw_t
 * are the packed forms (cvt_conv_weights_pack, taps 9 and 3) of w_s and w_t,
 * 16-byte aligned; the same kernels and y bit for bit as cvt_upsample3d,
 * without its two per-call repacks.  Source: as cvt_upsample3d.
 * workspace: cvt_upsample3d_packed_workspace bytes (the intermediate only).
 * Errors: as cvt_upsample3d; CVT_E_ALIGN also for packed weights that are not
 * 16-byte aligned.
 */
size_t cvt_upsample3d_packed_workspace(int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time);
int cvt_upsample3d_packed(const void* x, const void* pw_s, const void* pw_t, const float* b_s, const float* b_t,
                          void* y, int B, int Cin, int Cout, int T, int H, int W, int up_space, int up_time,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * FSQ dequantize fused with the decoder's first layer, the 1x1 projection
 * D -> Cout: y = w_p . codes + b_p per position, the codes being those of
 * cvt_fsq_dequantize rounded to bf16, accumulated in float32 in channel order,
 * so y equals cvt_fsq_dequantize (bf16 NTHWC) followed by
 * cvt_causal_conv3d_fact with k = 1 bit for bit, without writing the codes.
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 7.2 (indices_to_codes
 * restores the codes from the index) and the model card's "Model Architecture"
 * (the decoder mirrors the encoder, whose last layer is the 1x1 projection).
 *
 * indices: int32 [B, T, H, W]; levels: host int32[D]; w_p: bf16 [Cout, D, 1, 1,
 * 1]; b_p: float32 [Cout] or NULL; y: bf16 NTHWC [B, Cout, T, H, W].  An index
 * outside [0, prod L) gives NaN outputs and, when d_invalid_count is not NULL,
 * is ADDED to that int32 device counter.
 * Errors: CVT_E_NULL, CVT_E_LEVELS (as cvt_fsq_quantize), CVT_E_SHAPE for a
 * non-positive size or Cout above 4096, CVT_E_ALIGN.
 */
int cvt_fsq_dequantize_proj(const int32_t* indices, const int32_t* levels, int D, const void* w_p, const float* b_p,
                            void* y, int B, int Cout, int T, int H, int W, int32_t* d_invalid_count, void* stream);

/*
 * Cross-stage fusion: the Haar patcher inside the first convolution.  Computes
 *   y = cvt_causal_conv3d_fact(cvt_haar3d_fwd(x, temporal_levels = 2), w_s, w_t)
 * for a 3-channel clip without writing the 192 Haar coefficient channels: the
 * spatial convolution computes them from the pixels while it stages its input
 * (each 4 x 4 x 4 block per pixel channel; by linearity of the transform in an
 * order of additions that differs from cvt_haar3d_fwd's, so values may differ
 * from the unfused route by a bf16 rounding step).
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 7.1 (the Haar
 * patcher is a fixed, parameter-free first stage of the encoder) and the
 * Cosmos-Predict1 summary, section "1) Cosmos Tokenizer" (the factorized causal
 * convolution that follows it).
 *
 * x:   bf16 NCTHW [B, 3, T, H, W], T = 1 + 4k, H and W multiples of 4, below
 *      2 GiB.
 * w_s: bf16 [Cout, 192, 1, 3, 3] over the coefficient channels in the order
 *      cvt_haar3d_fwd writes them; w_t: bf16 [Cout, Cout, 3, 1, 1] or NULL
 *      (spatial part only); b_s, b_t: float32 [Cout] or NULL.
 * y:   bf16 NTHWC [B, Cout, 1 + (T-1)/4, H/4, W/4].  64 <= Cout <= 4096,
 *      Cout % 8 == 0.
 * workspace: cvt_haar3d_conv3d_fact_workspace() bytes (parts: CVT_CONV_SPATIAL,
 *      or CVT_CONV_SPATIAL | CVT_CONV_TEMPORAL when w_t is given).
 * Errors: CVT_E_NULL (x, w_s, y), CVT_E_SHAPE (sizes above), CVT_E_ALIGN,
 *      CVT_E_WORKSPACE.
 */
size_t cvt_haar3d_conv3d_fact_workspace(int B, int Cout, int T, int H, int W, int parts);
int cvt_haar3d_conv3d_fact(const void* x, const void* w_s, const void* w_t, const float* b_s, const float* b_t,
                           void* y, int B, int Cout, int T, int H, int W, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Cross-stage fusion: FSQ dequantize and the decoder's 1x1 projection inside the
 * decoder's first convolution.  Computes
 *   y = cvt_causal_conv3d_fact(cvt_fsq_dequantize_proj(indices, w_lift), w_s, w_t)
 * without writing the Cmid-channel projection: the spatial convolution computes
 * it from the int32 index of each position while it stages its input, rounded
 * exactly as cvt_fsq_dequantize_proj rounds it, so y equals the unfused route
 * bit for bit.
 *
 * Defined by: "NVIDIA Cosmos Tokenizer 完全指南", section 7.2 (FSQ: codes come
 * from the index by mixed-radix digits, no codebook lookup) and the model card
 * "Model Architecture" (the decoder mirrors the encoder, so its first layers are
 * the projection out of the latent and the factorized causal convolution).
 *
 * indices: int32 [B, T, H, W] below 2 GiB; levels, D: as cvt_fsq_dequantize
 *      (an out-of-range index gives NaN codes; it is not counted here).
 * w_lift: bf16 [Cmid, D, 1, 1, 1], Cmid a multiple of 32 up to 256; b_lift:
 *      float32 [Cmid] or NULL.
 * w_s: bf16 [Cout, Cmid, 1, 3, 3]; w_t: bf16 [Cout, Cout, 3, 1, 1] or NULL;
 *      b_s, b_t: float32 [Cout] or NULL.  64 <= Cout <= 4096, Cout % 8 == 0.
 * y:   bf16 NTHWC [B, Cout, T, H, W].
 * workspace: cvt_fsq_dequantize_conv3d_fact_workspace() bytes (parts as for
 *      cvt_haar3d_conv3d_fact).
 * Errors: CVT_E_NULL, CVT_E_LEVELS, CVT_E_SHAPE, CVT_E_ALIGN, CVT_E_WORKSPACE.
 */
size_t cvt_fsq_dequantize_conv3d_fact_workspace(int B, int Cmid, int Cout, int T, int H, int W, int parts);
int cvt_fsq_dequantize_conv3d_fact(const int32_t* indices, const int32_t* levels, int D, const void* w_lift,
                                   const float* b_lift, const void* w_s, const void* w_t, const float* b_s,
                                   const float* b_t, void* y, int B, int Cmid, int Cout, int T, int H, int W,
                                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CVT_H */
