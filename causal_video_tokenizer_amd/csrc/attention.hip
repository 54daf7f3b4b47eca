// Factorized causal self-attention over an NTHWC bf16 feature map.
//
// The operation is the space-time factorized causal self-attention that
// "Cosmos World Foundation Model Platform for Physical AI (Cosmos-Predict1)",
// section "1) Cosmos Tokenizer", pairs with the factorized convolution, and the
// model card's "Model Architecture" calls causal temporal attention: per head
// (d = C / heads consecutive channels), softmax(Q K^T / sqrt(d)) V
//   * SPATIAL: over the H*W positions of one frame, every position attending to
//     every position of the frame;
//   * TEMPORAL: over the T frames of one position, causal (frame t sees s <= t).
// Q, K, V and the output are [B, C, T, H, W] bf16 in NTHWC order; scores,
// softmax and accumulation are fp32, the probabilities enter the P V product
// as bf16, the output is rounded to bf16 once.
//
// Kernels:
//   * attn_spatial_kernel<D> - flash attention (d = 32, 64, 128) on bf16 MFMA 32x32x16, in
//     transposed form: S^T = K Q^T and O^T = V^T P^T, so a lane owns one query
//     column of every accumulator and the running max / sum of the online
//     softmax stay in its registers (the two lane halves of a column exchange
//     once per block).  A lane's 16 S^T values of a 32-key block are keys
//     8 (r / 4) + 4 (lane / 32) + r % 4; bf16-rounded, the values r = 8h .. 8h+7
//     are directly the B operand of a 16-key k-step whose key order is that
//     permutation, and V^T is staged in LDS with its keys in the same order, so
//     P never leaves the registers.
//   * attn_temporal_mfma_kernel - causal attention with d = 64 and T <= 32: one wave
//     per (position, head) sequence, the T x T scores in one MFMA block; a few FLOPs
//     per byte, so it is bound by HBM, not by the matrix cores;
//   * attn_temporal_kernel - the other temporal cases (d = 32, or 32 < T, T * C <=
//     16384): K and V of a few consecutive positions staged in LDS (one contiguous run
//     per frame), one thread per (position, head, query frame) in fp32;
//   * attn_generic_kernel - every other shape of either axis (any head dim d % 8 == 0 up
//     to 256, any sequence length): one thread per query, keys and values from global
//     memory, fp32.
#include <algorithm>
#include <type_traits>

#include "cvt_internal.h"

namespace cvt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------------------
// Spatial attention, head dim D in {32, 64, 128}.  Workgroup = 4 waves x 32 QB queries
// (QB 32-query MFMA column blocks per wave: 2 up to D = 64, 1 at D = 128, whose
// accumulators are twice as many) of one (clip, frame, head) sequence; the keys go by in
// blocks of 64, staged in LDS (K rows [key][D channels], V^T rows [channel][64 keys] with
// their 16-byte chunks swizzled, 16-byte padded rows, two buffers), loaded during the
// previous block.  Per block and wave:
// 2 key blocks x QB query blocks x D/16 channel k-steps MFMAs for S^T and D/32 channel
// blocks x QB query blocks x 4 key k-steps for O^T.
constexpr int AKB = 64;              // keys per block
constexpr int AVRS = AKB * 2 + 16;   // bytes per V^T row in LDS

template <int D>
struct SpatialAttnCfg {
    static_assert(D == 32 || D == 64 || D == 128, "spatial head dims 32, 64, 128");
    static constexpr int QB = D <= 64 ? 2 : 1;   // 32-query blocks per wave
    static constexpr int QW = 32 * QB;           // queries per wave
    static constexpr int QT = 4 * QW;            // queries per workgroup
    static constexpr int KRS = D * 2 + 16;       // bytes per K row in LDS
    static constexpr int KBUF = AKB * KRS;
    static constexpr int VBUF = D * AVRS;
    static constexpr int CPK = D / 8;            // 16-byte chunks per key row
    static constexpr int KL = AKB * CPK / 256;   // K chunks per thread and block
    static constexpr int VI = 32 * CPK;          // V items: (key pair, chunk)
    static constexpr int VL = (VI + 255) / 256;  // V items per thread
    // V^T rows are swizzled in 16-byte chunks: row r keeps chunk k at k ^ (((r / 16) * SW) % 8),
    // which makes both the staging writes (4-byte key pairs of 8 channels per lane) and the
    // fragment reads (16 rows per 16 lanes) free of bank conflicts (d = 32, 64; d = 128: the
    // writes 2-way instead of 8-way)
    static constexpr int SW = D == 32 ? 4 : 2;
};

struct AttnGeom {
    int N;          // tokens per sequence (H * W)
    int C;          // channels per token
    int G;          // heads
    int nqt;        // query tiles per sequence
    int ntiles, per_xcd;
    int ext;        // bytes from a sequence's first element to its last (buffer extent)
    float scale2;   // log2(e) / sqrt(d)
};

// 2^x by the hardware's v_exp_f32 alone.  exp2f adds a denormal-range rescaling (compares,
// selects and an ldexp around every exponential) that a softmax does not need: a weight
// below 2^-126 next to the row maximum's weight of 1 is zero either way.  2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// Position of key k within its 16-key group in a V^T row: lane half h's keys of a k-step,
// {4h .. 4h+3, 8+4h .. 8+4h+3}, become the contiguous 8 at 8h (bits 2 and 3 swapped).
__device__ __forceinline__ int vperm(int k) {
    return (k & ~15) | (k & 3) | (((k >> 3) & 1) << 2) | (((k >> 2) & 1) << 3);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_spatial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, AttnGeom g) {
    using Cf = SpatialAttnCfg<D>;
    constexpr int QB = Cf::QB, QW = Cf::QW, QT = Cf::QT, KRS = Cf::KRS, KBUF = Cf::KBUF, VBUF = Cf::VBUF;
    constexpr int CPK = Cf::CPK, KL = Cf::KL, VI = Cf::VI, VL = Cf::VL, CB = D / 32;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (KBUF + VBUF)];
    // XCD-aware order: consecutive tiles (the query tiles of one sequence, which read the
    // same keys) run on one XCD's L2
    const int tile = (int)(blockIdx.x & 7) * g.per_xcd + (int)(blockIdx.x >> 3);
    if (tile >= g.ntiles) return;
    const int qt = tile % g.nqt, seq = tile / g.nqt;
    const int head = seq % g.G;
    const long long base = (long long)(seq / g.G) * g.N * g.C + head * D;  // element offset of token 0
    const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + base), (short)0, g.ext, 0x00020000);
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), (short)0, g.ext, 0x00020000);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), (short)0, g.ext, 0x00020000);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int px = lane & 31, hh = lane >> 5;
    const int rowb = g.C * 2;  // bytes between consecutive tokens

    // Q^T B operand: lane (query px of block qb, half hh) holds channels 16 ks + 8 hh .. +7.
    // Queries past N read zeros (past the buffer) and are never stored.
    bf16x8_t qf[QB][D / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = qt * QT + wave * QW + qb * 32 + px;
        const int off = qi < g.N ? qi * rowb : 0x7fffff00;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[qb][ks] = __builtin_bit_cast(bf16x8_t,
                                            __builtin_amdgcn_raw_buffer_load_b128(qres, off + (ks * 16 + hh * 8) * 2, 0, 0));
    }

    // Staging of a key block: K chunk i = tid + 256 r is key i / CPK at 16-byte chunk i % CPK;
    // V item i is the key pair 2 p, 2 p + 1 (p = i / CPK) at chunk i % CPK.  Keys past N are
    // staged as zeros (and masked from the scores).
    uint4 kst[KL], vst[VL][2];
    auto load_block = [&](int blk) {
#pragma unroll
        for (int r = 0; r < KL; ++r) {
            const int i = tid + 256 * r, j = blk * AKB + i / CPK, c = i % CPK;
            const auto kv = __builtin_amdgcn_raw_buffer_load_b128(kres, j < g.N ? j * rowb + c * 16 : 0x7fffff00, 0, 0);
            kst[r] = *reinterpret_cast<const uint4*>(&kv);
        }
#pragma unroll
        for (int r = 0; r < VL; ++r) {
            const int i = tid + 256 * r, p = i / CPK, c = i % CPK;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int jv = blk * AKB + 2 * p + e;
                const auto vv = __builtin_amdgcn_raw_buffer_load_b128(
                    vres, i < VI && jv < g.N ? jv * rowb + c * 16 : 0x7fffff00, 0, 0);
                vst[r][e] = *reinterpret_cast<const uint4*>(&vv);
            }
        }
    };
    auto store_block = [&](int buf) {
        uint8_t* sk = smem + buf * (KBUF + VBUF);
        uint8_t* sv = sk + KBUF;
#pragma unroll
        for (int r = 0; r < KL; ++r) {
            const int i = tid + 256 * r;
            *reinterpret_cast<uint4*>(sk + (i / CPK) * KRS + (i % CPK) * 16) = kst[r];
        }
#pragma unroll
        for (int r = 0; r < VL; ++r) {
            const int i = tid + 256 * r, p = i / CPK, c = i % CPK;
            if (VI % 256 == 0 || i < VI) {
                // V^T: channel c * 8 + e gets the pair (key 2 p, key 2 p + 1) at its permuted column
                const uint32_t a[4] = {vst[r][0].x, vst[r][0].y, vst[r][0].z, vst[r][0].w};
                const uint32_t b[4] = {vst[r][1].x, vst[r][1].y, vst[r][1].z, vst[r][1].w};
                // byte column of the key pair, its 16-byte chunk swizzled by the rows' group (all
                // 8 rows c * 8 .. c * 8 + 7 of the chunk lie in one 16-row group)
                const int col = (vperm(2 * p) * 2) ^ ((((c >> 1) * Cf::SW) & 7) << 4);
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    // channels 2 e2 and 2 e2 + 1 of the chunk: low halves, then high halves
                    *reinterpret_cast<uint32_t*>(sv + (c * 8 + 2 * e2) * AVRS + col) = (a[e2] & 0xffffu) | (b[e2] << 16);
                    *reinterpret_cast<uint32_t*>(sv + (c * 8 + 2 * e2 + 1) * AVRS + col) =
                        (a[e2] >> 16) | (b[e2] & 0xffff0000u);
                }
            }
        }
    };

    f32x16_t o[CB][QB];  // O^T: [channel block][query block]
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[cb][qb][e] = 0.0f;
    float m[QB], lp[QB];  // running max (log2 domain) and the sum over the lane's own keys
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        lp[qb] = 0.0f;
    }

    const int nblk = (g.N + AKB - 1) / AKB;
    // per-lane byte offsets of the K and V^T fragments within a buffer; every fragment is
    // this plus a compile-time offset
    const int klane = px * KRS + hh * 16, vlane = KBUF + px * AVRS + hh * 16;
    // V^T fragment (channel block cb, keys 32 kb + 16 h2 + 8 hh ..): row cb * 32 + px, chunk
    // 4 kb + 2 h2 + hh swizzled by ((row / 16) * SW) % 8 = (cb * 2 SW) % 8 ^ (px / 16) SW
    // (even: the lane's hh bit stays); vsw[j] = byte offset of chunk pair 2 j after the lane's part
    int vsw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vsw[j] = ((2 * j) ^ (((px >> 4) * Cf::SW) & 7)) * 16;
    auto vfrag = [&](const uint8_t* vb, int cb, int kb, int h2) {  // vb: the buffer's base + vlane
        const int k2 = (4 * kb + 2 * h2) ^ ((cb * 2 * Cf::SW) & 7);  // compile-time
        return *reinterpret_cast<const bf16x8_t*>(vb + cb * 32 * AVRS + vsw[k2 >> 1]);
    };

    // One key block.  MASKED (the last block when N is not a multiple of 64): keys past N
    // get a score of -inf.  A compile-time flag, so that the full blocks carry no mask code.
    auto block = [&](int blk, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const uint8_t* kbase = smem + (blk & 1) * (KBUF + VBUF) + klane;
        const uint8_t* vbase = smem + (blk & 1) * (KBUF + VBUF) + vlane;
        if (blk + 1 < nblk) load_block(blk + 1);

        // S^T = K Q^T: rows = 64 keys (2 blocks), columns = the wave's queries; the first
        // k-step accumulates onto the inline constant 0 (no register clearing per block)
        f32x16_t s[2][QB];
        const f32x16_t zero16 = {};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kbase + kb * 32 * KRS + ks * 32);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], ks == 0 ? zero16 : s[kb][qb],
                                                                         0, 0, 0);
            }
        }
        if constexpr (MASKED) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = blk * AKB + kb * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
                    if (j >= g.N) {
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = -INFINITY;
                    }
                }
        }

        // online softmax per query column; P (bf16) straight into the P V MFMAs
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[qb], mx * g.scale2);
            const float alpha = fast_exp2(m[qb] - mnew);
            m[qb] = mnew;
            // the row sum adds the bf16-rounded weights that enter the P V product (two per
            // v_dot2_f32_bf16), so numerator and denominator use the same weights
            float sum = 0.0f;
            bf16x8_t pf[2][2];  // [key block][half of the block]
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(s[kb][qb][8 * h2 + e], g.scale2, -mnew));
                    uint32_t u[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        u[e2] = pack_bf16x2(p[2 * e2], p[2 * e2 + 1]);
                        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e2]), ones, sum, false);
                    }
                    pf[kb][h2] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
                }
            lp[qb] = lp[qb] * alpha + sum;
            // rescale the accumulators only when some lane's running maximum moved (alpha < 1);
            // once the maximum has settled, most blocks skip it
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[cb][qb][e] *= alpha;
            }
            // O^T += V^T P^T: A = V^T rows (32 channels) x the k-step's 16 keys in lane order
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const bf16x8_t vf = vfrag(vbase, cb, kb, h2);
                        o[cb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][h2], o[cb][qb], 0, 0, 0);
                    }
        }
        if (blk + 1 < nblk) store_block((blk + 1) & 1);
        __syncthreads();
    };

    load_block(0);
    store_block(0);
    __syncthreads();
    const int nfull = g.N / AKB;  // blocks without keys past N
    for (int blk = 0; blk < nfull; ++blk) block(blk, std::false_type{});
    if (nfull < nblk) block(nfull, std::true_type{});

    // normalise and store: element r of O^T block (cb, qb) is channel 32 cb + 8 (r / 4) +
    // 4 hh + r % 4 of the lane's query; four consecutive channels per 8-byte store
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = lp[qb] + __shfl_xor(lp[qb], 32);
        const float inv = 1.0f / l;
        const int qi = qt * QT + wave * QW + qb * 32 + px;
        if (qi < g.N) {
            uint16_t* orow = O + base + (long long)qi * g.C;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    uint2 u;
                    u.x = pack_bf16x2(o[cb][qb][4 * q4] * inv, o[cb][qb][4 * q4 + 1] * inv);
                    u.y = pack_bf16x2(o[cb][qb][4 * q4 + 2] * inv, o[cb][qb][4 * q4 + 3] * inv);
                    *reinterpret_cast<uint2*>(orow + cb * 32 + q4 * 8 + hh * 4) = u;
                }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Temporal causal attention.  Workgroup = NP consecutive positions of one clip, all heads,
// all T frames: K and V are read as one contiguous run of NP * C * 2 bytes per frame and
// staged in LDS (layout below), then thread -> (position, head, query frame t).  Each
// computes its query's softmax over frames 0..t in two passes (the
// maximum, then the weights and the weighted sum; the scores are bf16 dot products on the
// packed inputs, v_dot2_f32_bf16 with fp32 accumulation; weights and sums in fp32) and
// writes its d output channels.
// K and V rows in LDS: [frame][position][head][D + 8] (a head row padded by 16 bytes, so
// the rows of 16 consecutive (position, head) pairs start on 16 distinct 4-bank groups and
// a wave's reads of one key frame are conflict-free).  80 KB: two workgroups per CU.
constexpr int TLDS = 81920;

struct TAttnGeom {
    int B, T, HW, C, G;
    int np;        // positions per workgroup
    int ntp;       // position tiles per clip
    float scale2;  // log2(e) / sqrt(d)
};

template <int D>
__global__ __launch_bounds__(256) void attn_temporal_kernel(const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V,
                                                            uint16_t* __restrict__ O, TAttnGeom g) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[TLDS];
    const int b = blockIdx.x / g.ntp, p0 = (blockIdx.x % g.ntp) * g.np;
    const int np = min(g.np, g.HW - p0);  // positions in this tile
    constexpr int DP = D + 8;             // padded head row (elements)
    const int prow = g.G * DP;            // elements per (frame, position) in LDS
    const int frow = np * prow;           // elements per frame in LDS
    uint16_t* sk = reinterpret_cast<uint16_t*>(smem);
    uint16_t* sv = sk + g.T * g.np * prow;
    const size_t fstride = (size_t)g.HW * g.C;  // elements between frames in memory
    const size_t tbase = ((size_t)b * g.T * g.HW + p0) * g.C;
    // stage K and V: 16-byte chunks of each frame's contiguous run of np * C elements,
    // eight chunks of each tensor per thread in flight before any is stored
    const int cpp = g.C / 8;   // chunks per position
    const int cpr = np * cpp;  // chunks per frame run
    const int nch = g.T * cpr;
    for (int q0 = 0; q0 < nch; q0 += 8 * 256) {
        uint4 kr[8], vr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = min(q0 + i * 256 + (int)threadIdx.x, nch - 1);  // clamped: re-reads a valid chunk
            const int t = q / cpr, c = q - t * cpr;
            const size_t src = tbase + t * fstride + (size_t)c * 8;
            kr[i] = ld_stream16(K + src);
            vr[i] = ld_stream16(V + src);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = q0 + i * 256 + (int)threadIdx.x;
            if (q < nch) {
                const int t = q / cpr, c = q - t * cpr;
                const int pl = c / cpp, ch = (c - pl * cpp) * 8;  // position, first channel
                const int dst = t * frow + pl * prow + (ch / D) * DP + ch % D;
                *reinterpret_cast<uint4*>(sk + dst) = kr[i];
                *reinterpret_cast<uint4*>(sv + dst) = vr[i];
            }
        }
    }
    __syncthreads();

    // thread -> (query frame t, head, position), t slowest: the lanes of a wave share t or
    // neighbouring t, so their causal loops (frames 0..t) have nearly equal lengths
    const int items = np * g.G * g.T, npg = np * g.G;
    for (int it = threadIdx.x; it < items; it += 256) {
        const int t = it / npg, rest = it - t * npg;
        const int hd = rest % g.G, pl = rest / g.G;
        const size_t tok = tbase + t * fstride + (size_t)pl * g.C + hd * D;
        bf16x2_t q2[D / 2];  // the query as bf16 pairs, the operands of v_dot2_f32_bf16
#pragma unroll
        for (int c = 0; c < D; c += 8) {
            const uint4 u = ld_stream16(Q + tok + c);
            q2[c / 2] = __builtin_bit_cast(bf16x2_t, u.x); q2[c / 2 + 1] = __builtin_bit_cast(bf16x2_t, u.y);
            q2[c / 2 + 2] = __builtin_bit_cast(bf16x2_t, u.z); q2[c / 2 + 3] = __builtin_bit_cast(bf16x2_t, u.w);
        }
        const int koff = pl * prow + hd * DP;
        auto score = [&](int j) {  // q . k_j in fp32, two products per instruction
            const uint16_t* kr = sk + j * frow + koff;
            float a = 0.0f;
#pragma unroll
            for (int c = 0; c < D; c += 8) {
                const uint4 u = *reinterpret_cast<const uint4*>(kr + c);
                a = __builtin_amdgcn_fdot2_f32_bf16(q2[c / 2], __builtin_bit_cast(bf16x2_t, u.x), a, false);
                a = __builtin_amdgcn_fdot2_f32_bf16(q2[c / 2 + 1], __builtin_bit_cast(bf16x2_t, u.y), a, false);
                a = __builtin_amdgcn_fdot2_f32_bf16(q2[c / 2 + 2], __builtin_bit_cast(bf16x2_t, u.z), a, false);
                a = __builtin_amdgcn_fdot2_f32_bf16(q2[c / 2 + 3], __builtin_bit_cast(bf16x2_t, u.w), a, false);
            }
            return a;
        };
        // pass 1: the maximum score over frames 0..t, so pass 2 needs no rescaling
        float mx = -INFINITY;
        for (int j = 0; j <= t; ++j) mx = fmaxf(mx, score(j));
        const float m2 = mx * g.scale2;
        // pass 2: weights p_j = 2^(s_j c - m c) in fp32 and o += p_j v_j (each channel on its
        // own, so a non-finite value stays in its channel)
        float o[D];
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = 0.0f;
        float l = 0.0f;
        for (int j = 0; j <= t; ++j) {
            const float p = fast_exp2(fmaf(score(j), g.scale2, -m2));
            l += p;
            const uint16_t* vr = sv + j * frow + koff;
#pragma unroll
            for (int c = 0; c < D; c += 8) {
                const uint4 u = *reinterpret_cast<const uint4*>(vr + c);
                o[c] = fmaf(p, bf16_lo(u.x), o[c]); o[c + 1] = fmaf(p, bf16_hi(u.x), o[c + 1]);
                o[c + 2] = fmaf(p, bf16_lo(u.y), o[c + 2]); o[c + 3] = fmaf(p, bf16_hi(u.y), o[c + 3]);
                o[c + 4] = fmaf(p, bf16_lo(u.z), o[c + 4]); o[c + 5] = fmaf(p, bf16_hi(u.z), o[c + 5]);
                o[c + 6] = fmaf(p, bf16_lo(u.w), o[c + 6]); o[c + 7] = fmaf(p, bf16_hi(u.w), o[c + 7]);
            }
        }
        const float inv = 1.0f / l;
#pragma unroll
        for (int c = 0; c < D; c += 8) {
            uint4 u;
            u.x = pack_bf16x2(o[c] * inv, o[c + 1] * inv);
            u.y = pack_bf16x2(o[c + 2] * inv, o[c + 3] * inv);
            u.z = pack_bf16x2(o[c + 4] * inv, o[c + 5] * inv);
            u.w = pack_bf16x2(o[c + 6] * inv, o[c + 7] * inv);
            st_stream16(O + tok + c, u);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Temporal causal attention on the matrix cores (head dim 64, T <= 32): one wave per
// (clip, position, head) sequence, a workgroup = 4 consecutive sequences (with 4 heads, the
// 4 heads of one position, whose frame rows are one contiguous 512-byte run per frame).
// S^T = K Q^T is one 32 x 32 block (4 MFMAs over the channels; frames past T read zeros),
// keys after the query's frame are masked, the softmax runs over the lane's query column
// as in the spatial kernel, and O^T = V^T P^T takes 2 channel blocks x 2 key k-steps.  V^T
// goes through a wave-private LDS tile (64 channel rows of 32 keys in the k-step key order,
// 16-byte padded rows), Q, K and O through a wave-private tile of frame rows; 9.5 KB of LDS
// and at most 128 VGPRs per wave up to 24 frames, so 16 waves fit on a CU to hide HBM latency.
constexpr int TM_VRS = 32 * 2 + 16;  // bytes per V^T row (32 keys)
constexpr int TM_WAVE_LDS = 64 * TM_VRS;

struct TAttnMGeom {
    int T, HW, C, G;
    int nseq;       // sequences = B * HW * G
    int ext;        // bytes from a sequence's first element to its last (buffer extent)
    int fsb;        // bytes between frames
    float scale2;   // log2(e) / 8
};

// The waves loop over sequences (the grid-stride keeps the four waves of a workgroup on the
// four heads of one position, i.e. one contiguous 512-byte run per frame and tensor) and
// issue the next sequence's loads before computing the current one, so every wave keeps
// loads in flight through its compute phase.  A load instruction covers 8 whole frame rows
// (8 lanes x 16 bytes = the head's 128 bytes of a frame), NF = ceil(T / 8) per tensor; Q and
// K reach the MFMA operand layout through the wave's row tile in LDS (frame f at f * 144
// bytes), V through its V^T tile.
constexpr int TM_RRS = 64 * 2 + 16;            // bytes per staged frame row (64 channels)
constexpr int TM_ROWS_LDS = 32 * TM_RRS;       // the wave's Q / K row tile (32 frames)
template <int NF>
__global__ __launch_bounds__(256) void attn_temporal_mfma_kernel(const uint16_t* __restrict__ Q,
                                                                 const uint16_t* __restrict__ K,
                                                                 const uint16_t* __restrict__ V,
                                                                 uint16_t* __restrict__ O, TAttnMGeom g) {
    static_assert(NF >= 1 && NF <= 4, "T <= 32");
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * (TM_WAVE_LDS + TM_ROWS_LDS)];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int stride = (int)gridDim.x * 4;
    int sq = (int)blockIdx.x * 4 + wave;
    if (sq >= g.nseq) return;  // wave-uniform; the kernel has no workgroup barrier
    const int px = lane & 31, hh = lane >> 5;
    const int fr8 = lane >> 3, c8 = lane & 7;  // loads: frame 8 it + fr8, channels 8 c8 .. 8 c8 + 7
    const int per_b = g.HW * g.G;
    auto seq_base = [&](int s) {
        const int b = s / per_b, rem = s - b * per_b;
        const int pos = rem / g.G, head = rem - pos * g.G;
        return ((long long)b * g.T * g.HW + pos) * g.C + head * 64;  // frame 0 token
    };
    // frames past T, and every offset past the last sequence (the final prefetch), read
    // zeros from past the buffer with no memory access; the loads stay unconditional so that
    // the wait before a sequence's MFMAs covers only its own loads, not the prefetch after them
    auto load = [&](int s, uint4 (&qr)[NF], uint4 (&kr)[NF], uint4 (&vr)[NF]) {
        const bool live = s < g.nseq;
        const long long base = seq_base(live ? s : 0);
        const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + base), (short)0, g.ext, 0x00020000);
        const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), (short)0, g.ext, 0x00020000);
        const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), (short)0, g.ext, 0x00020000);
#pragma unroll
        for (int it = 0; it < NF; ++it) {
            const int fr = it * 8 + fr8;
            const int off = live && fr < g.T ? fr * g.fsb + c8 * 16 : 0x7fffff00;
            const auto qv = __builtin_amdgcn_raw_buffer_load_b128(qres, off, 0, 0);
            const auto kv = __builtin_amdgcn_raw_buffer_load_b128(kres, off, 0, 0);
            const auto vv = __builtin_amdgcn_raw_buffer_load_b128(vres, off, 0, 0);
            qr[it] = *reinterpret_cast<const uint4*>(&qv);
            kr[it] = *reinterpret_cast<const uint4*>(&kv);
            vr[it] = *reinterpret_cast<const uint4*>(&vv);
        }
    };
    uint8_t* vt = smem + wave * (TM_WAVE_LDS + TM_ROWS_LDS);
    uint8_t* rt = vt + TM_WAVE_LDS;
    // frames NF * 8 .. 31 of the row tile and keys past NF * 8 in V^T are never written:
    // zeros once (keys past T must be finite, their weights are 0)
    for (int i = lane; i < (TM_WAVE_LDS + TM_ROWS_LDS) / 16; i += 64)
        reinterpret_cast<uint4*>(vt)[i] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the MFMA operand of a row tile: lane (px, hh) holds frame px, channels 16 ks + 8 hh .. +7
    auto stage_rows = [&](const uint4 (&r)[NF], bf16x8_t (&f)[4]) {
#pragma unroll
        for (int it = 0; it < NF; ++it)
            *reinterpret_cast<uint4*>(rt + (it * 8 + fr8) * TM_RRS + c8 * 16) = r[it];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            f[ks] = *reinterpret_cast<const bf16x8_t*>(rt + px * TM_RRS + (ks * 16 + hh * 8) * 2);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the reads before the tile's next writes
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    uint4 qr[NF], kr[NF], vr[NF];
    load(sq, qr, kr, vr);
    for (;;) {
        const int nx = sq + stride;
        uint4 qn[NF], kn[NF], vn[NF];
        load(nx, qn, kn, vn);
        bf16x8_t qf[4], kf[4];
        stage_rows(qr, qf);
        stage_rows(kr, kf);
        // V^T into the wave's LDS tile: channel 8 c8 + e, key fr at its k-step column (the
        // tile is wave-private and its accesses execute in order: the previous sequence's
        // reads are done)
#pragma unroll
        for (int it = 0; it < NF; ++it) {
            // rows 16 .. 31 and 48 .. 63 (channel groups c8 = 2, 3, 6, 7) keep their two 32-byte
            // halves swapped: the 2-byte writes of a store then spread over twice the banks
            const int col = (vperm(it * 8 + fr8) * 2) ^ (((c8 >> 1) & 1) << 5);
            const uint32_t w[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int row = c8 * 8 + 2 * e2;
                *reinterpret_cast<uint16_t*>(vt + row * TM_VRS + col) = (uint16_t)(w[e2] & 0xffffu);
                *reinterpret_cast<uint16_t*>(vt + (row + 1) * TM_VRS + col) = (uint16_t)(w[e2] >> 16);
            }
        }
        // S^T = K Q^T (rows = keys, columns = queries)
        f32x16_t st;
#pragma unroll
        for (int e = 0; e < 16; ++e) st[e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], st, 0, 0, 0);
        // causal mask: key j after query px (this also masks keys past T for queries < T)
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = 8 * (r / 4) + 4 * hh + (r % 4);
            if (j > px) st[r] = -INFINITY;
            mx = fmaxf(mx, st[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m2 = mx * g.scale2;
        float sum = 0.0f;
        bf16x8_t pf[2];
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            uint32_t u[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = fast_exp2(fmaf(st[8 * h2 + 2 * e2], g.scale2, -m2));
                const float p1 = fast_exp2(fmaf(st[8 * h2 + 2 * e2 + 1], g.scale2, -m2));
                u[e2] = pack_bf16x2(p0, p1);
                sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e2]), ones, sum, false);
            }
            pf[h2] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
        }
        const float l = sum + __shfl_xor(sum, 32);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x16_t ot[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) ot[cb][e] = 0.0f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const bf16x8_t vf =
                    *reinterpret_cast<const bf16x8_t*>(vt + (cb * 32 + px) * TM_VRS + ((h2 ^ (px >> 4)) * 16 + hh * 8) * 2);
                ot[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[h2], ot[cb], 0, 0, 0);
            }
        }
        {
            // O rows staged in the row tile (frame px at byte px * 144), then written as
            // 16-byte pieces, 8 lanes per 128-byte frame row, with streaming stores (written
            // once, read by the next layer)
            const float inv = 1.0f / l;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    uint2 u;
                    u.x = pack_bf16x2(ot[cb][4 * q4] * inv, ot[cb][4 * q4 + 1] * inv);
                    u.y = pack_bf16x2(ot[cb][4 * q4 + 2] * inv, ot[cb][4 * q4 + 3] * inv);
                    *reinterpret_cast<uint2*>(rt + px * TM_RRS + (cb * 32 + q4 * 8 + hh * 4) * 2) = u;
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint16_t* obase = O + seq_base(sq);
#pragma unroll
            for (int it = 0; it < NF; ++it) {
                const int fr = it * 8 + fr8;
                const uint4 v = *reinterpret_cast<const uint4*>(rt + fr * TM_RRS + c8 * 16);
                if (fr < g.T) st_stream16(obase + (long long)fr * (g.fsb / 2) + c8 * 8, v);
            }
        }
        if (nx >= g.nseq) break;
        sq = nx;
#pragma unroll
        for (int it = 0; it < NF; ++it) {
            qr[it] = qn[it];
            kr[it] = kn[it];
            vr[it] = vn[it];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // this sequence's tile reads before the next writes
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <int D>
hipError_t launch_temporal(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int B, int C, int T,
                           int HW, int G, hipStream_t s) {
    TAttnGeom g{};
    g.B = B; g.T = T; g.HW = HW; g.C = C; g.G = G;
    g.np = TLDS / (2 * T * (C + 8 * G) * 2);  // at least 1: T * C <= 16384 and C + 8 G <= 1.25 C
    if (g.np > HW) g.np = HW;
    g.ntp = (HW + g.np - 1) / g.np;
    g.scale2 = 1.4426950408889634f / sqrtf((float)D);
    const long long nblk = (long long)B * g.ntp;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_temporal_kernel<D>), dim3((unsigned)nblk), dim3(256), 0, s, q, k, v, o, g);
    return hipGetLastError();
}

}  // namespace

int attention_max_tc() { return 16384; }

// ---------------------------------------------------------------------------------------
// Any head dim (d % 8 == 0, d <= 256) and any sequence length, either axis: one thread per
// (sequence, query token), keys and values read straight from global memory (the
// sequence's rows are shared by the wave's threads through the caches), two passes: the
// maximum score, then, for each 64-channel slice of the output, the weights (fp32) and the
// weighted sum of the values, the scores recomputed per slice.  The path for the shapes the
// tiled kernels do not take (spatial head dims other than 32, 64, 128; temporal head dims
// other than 32, 64 or sequences whose K and V do not fit the LDS tile); its rate is not a
// target.
struct GAttnGeom {
    long long nitems;    // sequences x tokens
    int N;               // tokens per sequence
    int G, d, C, HW, T;  // heads, head dim, channels, positions per frame, frames
    int causal;          // temporal: token i sees tokens j <= i
    long long tstride;   // elements between consecutive tokens of a sequence
    float scale2;        // log2(e) / sqrt(d)
};

__global__ __launch_bounds__(256) void attn_generic_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V,
                                                           uint16_t* __restrict__ O, GAttnGeom g) {
    const long long item = (long long)blockIdx.x * 256 + threadIdx.x;
    if (item >= g.nitems) return;
    const long long sq = item / g.N;
    const int i = (int)(item - sq * g.N);
    const int head = (int)(sq % g.G);
    const long long outer = sq / g.G;  // spatial: clip * T + frame; temporal: clip * HW + position
    long long base;                    // element offset of the sequence's token 0
    if (g.causal) {
        const long long b = outer / g.HW, pos = outer - b * g.HW;
        base = (b * g.T * g.HW + pos) * g.C + (long long)head * g.d;
    } else {
        base = outer * g.N * g.C + (long long)head * g.d;
    }
    const uint16_t* qrow = Q + base + i * g.tstride;
    const int nk = g.causal ? i + 1 : g.N;
    auto score = [&](int j) {  // q . k_j in fp32, two products per instruction
        const uint16_t* krow = K + base + j * g.tstride;
        float a = 0.0f;
        for (int c = 0; c < g.d; c += 8) {
            const uint4 q = *reinterpret_cast<const uint4*>(qrow + c);
            const uint4 k = *reinterpret_cast<const uint4*>(krow + c);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x), a,
                                                false);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), a,
                                                false);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), a,
                                                false);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), a,
                                                false);
        }
        return a;
    };
    float mx = -INFINITY;
    for (int j = 0; j < nk; ++j) mx = fmaxf(mx, score(j));
    const float m2 = mx * g.scale2;
    for (int c0 = 0; c0 < g.d; c0 += 64) {
        const int nc = min(64, g.d - c0);  // a multiple of 8
        float o[64];
#pragma unroll
        for (int c = 0; c < 64; ++c) o[c] = 0.0f;
        float l = 0.0f;
        for (int j = 0; j < nk; ++j) {
            const float p = fast_exp2(fmaf(score(j), g.scale2, -m2));
            l += p;
            const uint16_t* vrow = V + base + j * g.tstride + c0;
#pragma unroll
            for (int c = 0; c < 64; c += 8) {
                if (c < nc) {
                    const uint4 u = *reinterpret_cast<const uint4*>(vrow + c);
                    o[c] = fmaf(p, bf16_lo(u.x), o[c]); o[c + 1] = fmaf(p, bf16_hi(u.x), o[c + 1]);
                    o[c + 2] = fmaf(p, bf16_lo(u.y), o[c + 2]); o[c + 3] = fmaf(p, bf16_hi(u.y), o[c + 3]);
                    o[c + 4] = fmaf(p, bf16_lo(u.z), o[c + 4]); o[c + 5] = fmaf(p, bf16_hi(u.z), o[c + 5]);
                    o[c + 6] = fmaf(p, bf16_lo(u.w), o[c + 6]); o[c + 7] = fmaf(p, bf16_hi(u.w), o[c + 7]);
                }
            }
        }
        const float inv = 1.0f / l;
        uint16_t* orow = O + base + i * g.tstride + c0;
#pragma unroll
        for (int c = 0; c < 64; c += 8) {
            if (c < nc) {
                uint4 u;
                u.x = pack_bf16x2(o[c] * inv, o[c + 1] * inv);
                u.y = pack_bf16x2(o[c + 2] * inv, o[c + 3] * inv);
                u.z = pack_bf16x2(o[c + 4] * inv, o[c + 5] * inv);
                u.w = pack_bf16x2(o[c + 6] * inv, o[c + 7] * inv);
                *reinterpret_cast<uint4*>(orow + c) = u;
            }
        }
    }
}

hipError_t launch_attention_generic(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O, int B, int C,
                                    int T, int HW, int heads, bool causal, hipStream_t s) {
    GAttnGeom g{};
    g.G = heads; g.d = C / heads; g.C = C; g.HW = HW; g.T = T;
    g.causal = causal ? 1 : 0;
    g.N = causal ? T : HW;
    g.tstride = causal ? (long long)HW * C : C;
    g.nitems = (long long)B * T * HW * heads;  // every (token, head) of the tensor is one query
    g.scale2 = 1.4426950408889634f / sqrtf((float)g.d);
    const long long nblk = (g.nitems + 255) / 256;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_generic_kernel, dim3((unsigned)nblk), dim3(256), 0, s, Q, K, V, O, g);
    return hipGetLastError();
}

template <int D>
hipError_t launch_spatial(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O, int B, int C, int T,
                          int HW, int heads, hipStream_t s) {
    using Cf = SpatialAttnCfg<D>;
    AttnGeom g{};
    g.N = HW; g.C = C; g.G = heads;
    g.nqt = (HW + Cf::QT - 1) / Cf::QT;
    const long long ntiles = (long long)B * T * heads * g.nqt;
    if (ntiles > 0x7ffffff0LL) return hipErrorInvalidConfiguration;
    g.ntiles = (int)ntiles;
    g.per_xcd = (int)((ntiles + 7) / 8);
    g.ext = ((HW - 1) * C + D) * 2;
    g.scale2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
    hipLaunchKernelGGL(attn_spatial_kernel<D>, dim3((unsigned)(8LL * g.per_xcd)), dim3(256), 0, s, Q, K, V, O, g);
    return hipGetLastError();
}

hipError_t launch_attention3d(const void* q, const void* k, const void* v, void* out, int B, int C, int T, int H,
                              int W, int heads, int axis, hipStream_t s) {
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    uint16_t* O = static_cast<uint16_t*>(out);
    const int d = C / heads, HW = H * W;
    if (axis == CVT_ATTN_SPATIAL) {
        switch (d) {
            case 32: return launch_spatial<32>(Q, K, V, O, B, C, T, HW, heads, s);
            case 64: return launch_spatial<64>(Q, K, V, O, B, C, T, HW, heads, s);
            case 128: return launch_spatial<128>(Q, K, V, O, B, C, T, HW, heads, s);
            default: return launch_attention_generic(Q, K, V, O, B, C, T, HW, heads, false, s);
        }
    }
    if ((d != 32 && d != 64) || (long long)T * C > attention_max_tc())
        return launch_attention_generic(Q, K, V, O, B, C, T, HW, heads, true, s);
    const long long fsb = (long long)HW * C * 2;         // bytes between frames
    const long long ext = (long long)(T - 1) * fsb + 64 * 2;  // a sequence's buffer extent
    const long long nseq = (long long)B * HW * heads;
    if (d == 64 && T <= 32 && ext < 0x7fff0000LL && nseq <= 0x7ffffff0LL) {
        TAttnMGeom g{};
        g.T = T; g.HW = HW; g.C = C; g.G = heads;
        g.nseq = (int)nseq;
        g.fsb = (int)fsb;
        g.ext = (int)ext;
        g.scale2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
        // persistent, each wave prefetching its next sequence: as many workgroups per CU as the
        // registers allow (up to 24 frames 128 VGPRs or fewer: four; 32 frames: three)
        const long long nwg = std::min((nseq + 3) / 4, 256LL * (T <= 24 ? 4 : 3));
        const dim3 grid((unsigned)nwg), block(256);
        switch ((T + 7) / 8) {
            case 1: hipLaunchKernelGGL(attn_temporal_mfma_kernel<1>, grid, block, 0, s, Q, K, V, O, g); break;
            case 2: hipLaunchKernelGGL(attn_temporal_mfma_kernel<2>, grid, block, 0, s, Q, K, V, O, g); break;
            case 3: hipLaunchKernelGGL(attn_temporal_mfma_kernel<3>, grid, block, 0, s, Q, K, V, O, g); break;
            default: hipLaunchKernelGGL(attn_temporal_mfma_kernel<4>, grid, block, 0, s, Q, K, V, O, g); break;
        }
        return hipGetLastError();
    }
    switch (d) {
        case 32: return launch_temporal<32>(Q, K, V, O, B, C, T, HW, heads, s);
        case 64: return launch_temporal<64>(Q, K, V, O, B, C, T, HW, heads, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace cvt
