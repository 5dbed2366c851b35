// quant.hip -- smoothing and quantisation kernels for gfx950 (HBM-bound).
//
// K mean (the smoothing of K): fp64 per-64-token-block channel sums, then an ordered
// fp64 sum over blocks; INT8 block quantisation of Q and smoothed K; the P.V operand
// V^ in FP16 or FP8-e4m3 with per-channel scales.  The arithmetic of each step is the
// one stated in include/sage.h (SageAttention project README, "Current Features":
// INT8 quantization and smoothing for QK^T, FP8 quantization for PV).  Every kernel
// walks a batch of sequences through a SeqMap, dense or packed (the variable-length
// form of the README's "Available APIs": sageattn_varlen); grids span the longest
// sequence and blocks past a sequence's end return at once.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace sage {

// ------------------------------------------------------------------------------------------
// K mean, pass 1: part[slot of block j][c] = sum of K[b,h,t,c] over the tokens t of
// block j, ascending, in fp64.  grid (max blocks, H, B), 256 threads: the block's
// 64 x D tile is read with coalesced 16-byte loads into LDS, then thread c < D walks
// its channel.
template <bool BF16, int DP, bool VEC8>
__device__ __forceinline__ void k_partial_block(const uint16_t* __restrict__ k, const SeqMap& m, int D,
                                                double* __restrict__ part, int j, int h, int b,
                                                uint16_t (*tile)[DP]) {
    constexpr int CH = DP / 8, RSTEP = 256 / CH;  // RSTEP token rows per pass
    const SeqView sv = seq_view(m, b, h);
    if (j * kBlk >= sv.n) return;  // the whole workgroup: past this sequence's end
    const int N = sv.n;
    const Strides st = m.st;
    const int ch = threadIdx.x % CH, r0 = threadIdx.x / CH, c0 = ch * 8;
    const uint16_t* base = k + sv.in_off;
#pragma unroll
    for (int p = 0; p < kBlk / RSTEP; p++) {
        const int tl = p * RSTEP + r0, t = j * kBlk + tl;
        v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < N && c0 < D) {
            const uint16_t* src = base + int64_t(t) * st.t + c0;
            if constexpr (VEC8) {
                r = *(const v8u16*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) r[e] = (c0 + e < D) ? src[e] : (unsigned short)0;
            }
        }
        *(v8u16*)&tile[tl][c0] = r;
    }
    __syncthreads();
    const int c = threadIdx.x;
    if (c >= D) return;
    const int nt = min(kBlk, N - j * kBlk);
    double s = 0.0;
    for (int t = 0; t < nt; t++) s += double(in_to_f32<BF16>(tile[t][c]));
    part[(sv.slot0 + j) * D + c] = s;
}
template <bool BF16, int DP, bool VEC8>
__global__ __launch_bounds__(256) void k_mean_partial_kernel(const uint16_t* __restrict__ k, SeqMap m, int D,
                                                             double* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kBlk][DP];
    k_partial_block<BF16, DP, VEC8>(k, m, D, part, blockIdx.x, blockIdx.y, blockIdx.z, tile);
}

// K mean, pass 2: mean = fp32((sum over blocks, ascending, of part) / N); 0 for a
// sequence without tokens.  One thread per (b, h, channel) in 64-thread workgroups
// (enough of them to spread over the CUs).
__global__ __launch_bounds__(64) void k_mean_final_kernel(const double* __restrict__ part, SeqMap m, int total,
                                                          int D, float* __restrict__ mean) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int c = i % D, h = (i / D) % m.H, b = i / (D * m.H);
    const SeqView sv = seq_view(m, b, h);
    const int nb = (sv.n + kBlk - 1) / kBlk;
    const double* p = part + sv.slot0 * D + c;
    double s = 0.0;
#pragma unroll 8
    for (int j = 0; j < nb; j++) s += p[int64_t(j) * D];
    mean[i] = sv.n > 0 ? float(s / double(sv.n)) : 0.0f;
}

// ------------------------------------------------------------------------------------------
// INT8 block quantisation.  One wave per 64-token block of one (b, head): grid
// (ceil(max blocks / 4), H, B), 4 waves per workgroup.  Lane l covers 8 consecutive
// channels (chunk l % CH, CH = Dp / 8) of the token rows l / CH + p * (64 / CH),
// p = 0 .. CH-1.  One scale per group of G tokens of the block:
//   y = x (Q) or fp32(x - mean[c]) (K); amax = max |y| over the group; scale =
//   amax / 127; inv = 127 / amax; code = clamp(rne(y * inv), -127, 127).
// G = 64: scale[slot]; G = 32: scale[2 slot + half]; G = 1: scale[row] (one per
// token: the rows of xq, padding rows 0).  G = 1 and 32 are the finer "per-thread"
// groups (SageAttention project README, "Project Updates" v2.0.1): a query column
// of the score MFMA per lane, the 32 keys of a half-wave.
// ROWMEAN: mean points at the (b, h) row of D means (for example in LDS), not at the
// [B][H][D] array.
template <bool BF16, int DP, bool VEC8, bool SMOOTH, int G = 64, bool ROWMEAN = false>
__device__ __forceinline__ void quant_block_wave(const uint16_t* __restrict__ x, const SeqMap& m, int D,
                                                 const float* __restrict__ mean, int8_t* __restrict__ xq,
                                                 float* __restrict__ scale, int j, int h, int b, int lane) {
    constexpr int CH = DP / 8;        // 8-channel chunks per row
    constexpr int RPP = kWave / CH;   // rows per pass
    constexpr int PASSES = kBlk / RPP;
    static_assert(G == 64 || G == 32 || G == 1, "token groups of 64, 32 or 1");
    const SeqView sv = seq_view(m, b, h);
    if (j * kBlk >= sv.n) return;  // this wave: past the sequence's end
    const int N = sv.n;
    const Strides st = m.st;
    const int64_t bh = int64_t(b) * m.H + h;
    const int ch = lane % CH, r0 = lane / CH;
    const int c0 = ch * 8;
    const uint16_t* base = x + sv.in_off;

    float mu[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
        mu[e] = (SMOOTH && c0 + e < D) ? mean[(ROWMEAN ? 0 : int64_t(bh) * D) + c0 + e] : 0.0f;

    v8u16 raw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; p++) {
        const int t = j * kBlk + p * RPP + r0;
        v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < N && c0 < D) {
            const uint16_t* src = base + int64_t(t) * st.t + c0;
            if constexpr (VEC8) {
                r = *(const v8u16*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) r[e] = (c0 + e < D) ? src[e] : (unsigned short)0;
            }
        }
        raw[p] = r;
    }
    auto yval = [&](int p, int e) {
        return SMOOTH ? in_to_f32<BF16>(raw[p][e]) - mu[e] : in_to_f32<BF16>(raw[p][e]);
    };
    // per-pass amax of this lane's real elements (a full block of whole chunks needs no
    // per-element test: channel padding holds y = 0)
    const bool full = VEC8 && (j + 1) * kBlk <= N;
    float am[PASSES];
    if (full) {
#pragma unroll
        for (int p = 0; p < PASSES; p++) {
            am[p] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; e++) am[p] = fmaxf(am[p], fabsf(yval(p, e)));
        }
    } else {
#pragma unroll
        for (int p = 0; p < PASSES; p++) {
            const int t = j * kBlk + p * RPP + r0;
            am[p] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; e++)
                if (t < N && c0 + e < D) am[p] = fmaxf(am[p], fabsf(yval(p, e)));
        }
    }
    // the amax of each pass's group
    if constexpr (G == 64) {
        float a = 0.0f;
#pragma unroll
        for (int p = 0; p < PASSES; p++) a = fmaxf(a, am[p]);
        a = wave_max(a);
#pragma unroll
        for (int p = 0; p < PASSES; p++) am[p] = a;
    } else if constexpr (G == 32) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int p = 0; p < PASSES; p++) {
            if (p * RPP < 32) a0 = fmaxf(a0, am[p]);
            else a1 = fmaxf(a1, am[p]);
        }
        a0 = wave_max(a0);
        a1 = wave_max(a1);
#pragma unroll
        for (int p = 0; p < PASSES; p++) am[p] = p * RPP < 32 ? a0 : a1;
    } else {
        // one row = CH consecutive lanes
#pragma unroll
        for (int p = 0; p < PASSES; p++)
#pragma unroll
            for (int o = CH / 2; o >= 1; o >>= 1) am[p] = fmaxf(am[p], __shfl_xor(am[p], o, 64));
    }
    // scale and inv once per group (the divisions are IEEE, so not cheap)
    float inv[PASSES];
    bool finite = true;
    auto group_scale = [&](float a, float& iv) {
        const bool zero = !(a > 0.0f);
        iv = zero ? 0.0f : 127.0f / a;
        finite = finite && a <= 3.4e38f && iv <= 3.4e38f;
        return zero ? 0.0f : a / 127.0f;
    };
    if constexpr (G == 1) {
#pragma unroll
        for (int p = 0; p < PASSES; p++) {
            const float sc = group_scale(am[p], inv[p]);
            if (ch == 0) scale[sv.row0 + j * kBlk + p * RPP + r0] = sc;
        }
    } else if constexpr (G == 32) {
        float i0, i1;
        const float s0 = group_scale(am[0], i0), s1 = group_scale(am[PASSES - 1], i1);
        if (lane == 0) {
            scale[(sv.slot0 + j) * 2] = s0;
            scale[(sv.slot0 + j) * 2 + 1] = s1;
        }
#pragma unroll
        for (int p = 0; p < PASSES; p++) inv[p] = p * RPP < 32 ? i0 : i1;
    } else {
        float i0;
        const float s0 = group_scale(am[0], i0);
        if (lane == 0) scale[sv.slot0 + j] = s0;
#pragma unroll
        for (int p = 0; p < PASSES; p++) inv[p] = i0;
    }
    if (full && __builtin_amdgcn_ballot_w64(!finite) == 0) {
        // Full block, whole 8-channel chunks, finite amax and inv everywhere (a
        // wave-uniform test): every element of the tile is real, channel padding reads
        // as x = 0 with mean 0, so y = 0 there.  |fp32(y * inv)| <= 127 (1 + 2^-23) by
        // construction, so the clamp is inert, and adding 1.5 * 2^23 rounds the product
        // to an integer (ties to even) held in the low mantissa bits: its low byte is
        // the two's-complement code.  Same codes as the general path below, at a
        // quarter of the instructions.
        constexpr float kRound = 12582912.0f;
#pragma unroll
        for (int p = 0; p < PASSES; p++) {
            uint32_t r[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float t = yval(p, e) * inv[p];
                r[e] = __float_as_uint(t + kRound);
            }
            // bytes 0 of r[0..3] and r[4..7] into one word each
            const uint32_t w0 = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u) |
                                __builtin_amdgcn_perm(r[3], r[2], 0x04000c0cu);
            const uint32_t w1 = __builtin_amdgcn_perm(r[5], r[4], 0x0c0c0400u) |
                                __builtin_amdgcn_perm(r[7], r[6], 0x04000c0cu);
            int8_t* dst = xq + (sv.row0 + j * kBlk + p * RPP + r0) * DP + c0;
            *(uint2*)dst = make_uint2(w0, w1);
        }
        return;
    }
#pragma unroll
    for (int p = 0; p < PASSES; p++) {
        const int t = j * kBlk + p * RPP + r0;
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            int code = 0;
            if (am[p] > 0.0f && t < N && c0 + e < D) {
                float r = rintf(yval(p, e) * inv[p]);
                // comparisons, not fminf/fmaxf: a NaN product stays NaN and converts to 0
                r = r > 127.0f ? 127.0f : r;
                r = r < -127.0f ? -127.0f : r;
                code = int(r);
            }
            w[e / 4] |= uint32_t(code & 0xff) << (8 * (e % 4));
        }
        int8_t* dst = xq + (sv.row0 + j * kBlk + p * RPP + r0) * DP + c0;
        *(uint2*)dst = make_uint2(w[0], w[1]);
    }
}
template <bool BF16, int DP, bool VEC8, bool SMOOTH, int G = 64>
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint16_t* __restrict__ x, SeqMap m, int D,
                                                           const float* __restrict__ mean, int8_t* __restrict__ xq,
                                                           float* __restrict__ scale) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    // smoothed K follows a pass that read K in ascending order: descending here, so the
    // blocks read last (still partly in the memory-side cache) come first
    const int bx = SMOOTH ? int(gridDim.x - 1 - blockIdx.x) : int(blockIdx.x);
    const int by = SMOOTH ? int(gridDim.y - 1 - blockIdx.y) : int(blockIdx.y);
    const int bz = SMOOTH ? int(gridDim.z - 1 - blockIdx.z) : int(blockIdx.z);
    quant_block_wave<BF16, DP, VEC8, SMOOTH, G>(x, m, D, mean, xq, scale, bx * 4 + wave, by, bz, lane);
}

// ------------------------------------------------------------------------------------------
// V operand, FP8 mode, pass 0: clear the per-channel amax buffer (a fill kernel rather
// than a memset so the sequence can be captured into a graph).
__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// FP8 pass 1: per-channel amax over all tokens of a sequence.  grid (ceil(max N/256),
// H, B), 256 threads; thread covers 8 channels of every (256 / CH)-th token of its
// 256-token slab.  The non-negative float maxima are combined with an integer atomic
// max on their bits.
template <bool BF16, int DP, bool VEC8>
__global__ __launch_bounds__(256) void v_amax_kernel(const uint16_t* __restrict__ v, SeqMap sm, int D,
                                                     uint32_t* __restrict__ amax_bits) {
    constexpr int CH = DP / 8, RSTEP = 256 / CH;
    __shared__ float red[RSTEP][DP];
    const int h = blockIdx.y, b = blockIdx.z;
    const SeqView sv = seq_view(sm, b, h);
    if (int(blockIdx.x) * 256 >= sv.n) return;  // the whole workgroup
    const int N = sv.n;
    const Strides st = sm.st;
    const int ch = threadIdx.x % CH, r0 = threadIdx.x / CH, c0 = ch * 8;
    const uint16_t* base = v + sv.in_off;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int t_end = min(N, int(blockIdx.x + 1) * 256);
    if (c0 < D) {
        // all loads of a round in flight at once; rows past the end read as 0, which
        // leaves a maximum of absolute values unchanged
        constexpr int ITER = 256 / RSTEP, ROUND = ITER < 16 ? ITER : 16;
#pragma unroll
        for (int i0 = 0; i0 < ITER; i0 += ROUND) {
            v8u16 r[ROUND];
#pragma unroll
            for (int u = 0; u < ROUND; u++) {
                const int t = blockIdx.x * 256 + r0 + (i0 + u) * RSTEP;
                r[u] = v8u16{0, 0, 0, 0, 0, 0, 0, 0};
                if (t < t_end) {
                    const uint16_t* src = base + int64_t(t) * st.t + c0;
                    if constexpr (VEC8) {
                        r[u] = *(const v8u16*)src;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; e++) r[u][e] = (c0 + e < D) ? src[e] : (unsigned short)0;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < ROUND; u++)
#pragma unroll
                for (int e = 0; e < 8; e++) m[e] = fmaxf(m[e], fabsf(in_to_f32<BF16>(r[u][e])));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) red[r0][c0 + e] = m[e];
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256) {
        float mx = 0.0f;
        for (int r = 0; r < RSTEP; r++) mx = fmaxf(mx, red[r][c]);
        atomicMax(amax_bits + (int64_t(b) * sm.H + h) * DP + c, __float_as_uint(mx));
    }
}

// ------------------------------------------------------------------------------------------
// Q, K and V together (sage_quant_qkv): the same results as the two-call path in four
// launches.  Pass 1 streams Q (block quantisation), K (block channel sums) and, in FP8
// mode, V (block channel maxima) side by side in one grid; pass 2 forms the K means
// and V maxima; pass 3 quantises K and V with the kernels above.  The per-block V
// maxima replace the integer atomics of v_amax_kernel (same maximum: max is exact in
// any order).  Sequences of at most kFoldBlocks blocks skip pass 2: the K and V
// launches reduce the partials of their own (b, kv head) in the same order (three
// launches in all).

// One 64-token K/V block of one (b, kv head): K channel sums as k_partial_block (fp64,
// ascending tokens) and, with VMAX, the per-channel maximum of |v| -> vpart[slot][c],
// c < DP (channel padding and rows past the end read as 0).  256 threads; the K tile
// goes to LDS and the V rows to registers with all loads in flight together.
template <bool BF16, int DP, bool VEC8, bool VMAX>
__device__ __forceinline__ void kv_stats_block(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               const SeqMap& m, int D, double* __restrict__ kpart,
                                               float* __restrict__ vpart, int j, int h, int b, uint16_t (*tile)[DP],
                                               float (*red)[DP]) {
    constexpr int CH = DP / 8, RSTEP = 256 / CH, ROWS = kBlk / RSTEP;
    const SeqView sv = seq_view(m, b, h);
    if (j * kBlk >= sv.n) return;  // the whole workgroup: past this sequence's end
    const int N = sv.n;
    const int ch = threadIdx.x % CH, r0 = threadIdx.x / CH, c0 = ch * 8;
    auto load8 = [&](const uint16_t* base, int t) {
        v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < N && c0 < D) {
            const uint16_t* src = base + int64_t(t) * m.st.t + c0;
            if constexpr (VEC8) {
                r = *(const v8u16*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) r[e] = (c0 + e < D) ? src[e] : (unsigned short)0;
            }
        }
        return r;
    };
    v8u16 kr[ROWS], vr[VMAX ? ROWS : 1];
#pragma unroll
    for (int u = 0; u < ROWS; u++) {
        const int t = j * kBlk + r0 + u * RSTEP;
        kr[u] = load8(k + sv.in_off, t);
        if constexpr (VMAX) vr[u] = load8(v + sv.in_off, t);
    }
#pragma unroll
    for (int u = 0; u < ROWS; u++) *(v8u16*)&tile[r0 + u * RSTEP][c0] = kr[u];
    if constexpr (VMAX) {
        float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < ROWS; u++)
#pragma unroll
            for (int e = 0; e < 8; e++) mx[e] = fmaxf(mx[e], fabsf(in_to_f32<BF16>(vr[u][e])));
#pragma unroll
        for (int e = 0; e < 8; e++) red[r0][c0 + e] = mx[e];
    }
    __syncthreads();
    const int c = threadIdx.x;
    if (c < D) {
        const int nt = min(kBlk, N - j * kBlk);
        double s = 0.0;
        for (int t = 0; t < nt; t++) s += double(in_to_f32<BF16>(tile[t][c]));
        kpart[(sv.slot0 + j) * D + c] = s;
    }
    if constexpr (VMAX) {
        for (int cc = c; cc < DP; cc += 256) {
            float a = 0.0f;
#pragma unroll
            for (int q = 0; q < RSTEP; q++) a = fmaxf(a, red[q][cc]);
            vpart[(sv.slot0 + j) * DP + cc] = a;
        }
    }
}

// Pass 2: per (b, kv head, channel): the K mean as k_mean_final_kernel (c < D) and, with
// VMAX, the V channel maximum over the sequence's blocks as float bits (c < DP), the
// form quant_v_kernel reads.  One thread per (b, kv head, c < DP).
template <int DP, bool VMAX>
__global__ __launch_bounds__(64) void qkv_pass2_kernel(const double* __restrict__ kpart,
                                                       const float* __restrict__ vpart, SeqMap m, int B, int D,
                                                       float* __restrict__ mean, uint32_t* __restrict__ amax_bits) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int c = i % DP, bh = i / DP;
    if (bh >= B * m.H) return;
    const int h = bh % m.H, b = bh / m.H;
    const SeqView sv = seq_view(m, b, h);
    const int nb = (sv.n + kBlk - 1) / kBlk;
    if (c < D) {
        const double* p = kpart + sv.slot0 * D + c;
        double s = 0.0;
#pragma unroll 32
        for (int j = 0; j < nb; j++) s += p[int64_t(j) * D];  // ascending block order
        mean[int64_t(bh) * D + c] = sv.n > 0 ? float(s / double(sv.n)) : 0.0f;
    }
    if constexpr (VMAX) {
        const float* p = vpart + sv.slot0 * DP + c;
        float a = 0.0f;
#pragma unroll 32
        for (int j = 0; j < nb; j++) a = fmaxf(a, p[int64_t(j) * DP]);
        amax_bits[int64_t(bh) * DP + c] = __float_as_uint(a);
    }
}

// V operand pass 2 (both modes): one workgroup per 64-token block.  Thread (q, ch)
// reads channels 8ch .. 8ch+7 of the four tokens 4q .. 4q+3 and writes, per channel,
// the four codes as one 4-byte (FP8) or 8-byte (FP16) word into a channel-major LDS
// tile, which then leaves in 16-byte stores ([Dp][64] per block).  Channel c's row
// sits at LDS row c ^ ((c >> 3) & 3) (FP8) or c ^ ((c >> 3) & 1) (FP16): the four
// (two) channel groups a wave writes at once then hit disjoint LDS banks.
//   FP16: v^ = fp16(clamp(v, +-65504)) (round half even).
//   FP8:  v^ = e4m3(clamp(fp32(v * inv[c]), +-448)), inv = fp32(448 / amax[c]);
//         the block-0 workgroup also writes v_scale[c] = fp32(amax[c] / 448).
// FOLD (FP8, short sequences): amax[c] is reduced here from the per-block channel maxima
// vpart of qkv_pass1_kernel, as qkv_pass2_kernel would (amax_bits is then unused).
// The body of quant_v_kernel for block j of (b, kv head h), run by NT >= 2 DP threads
// (threads from 2 DP on only help with the final copy and meet the barriers); tile is
// the workgroup's LDS tile of DP * 64 * (1 | 2) bytes, samax DP floats (FOLD).
template <bool BF16, int DP, bool VEC8, bool FP8, bool FOLD, int NT>
__device__ __forceinline__ void v_block(const uint16_t* __restrict__ v, const SeqMap& m, int D,
                                        const uint32_t* __restrict__ amax_bits, void* __restrict__ vhat,
                                        float* __restrict__ vscale, const float* __restrict__ vpart, int j, int h,
                                        int b, uint8_t* __restrict__ tile, float* __restrict__ samax) {
    constexpr int ELT = FP8 ? 1 : 2;
    constexpr int CH = DP / 8;               // 8-channel chunks per token row
    constexpr int THREADS = CH * (kBlk / 4);  // one thread per (token quad, chunk)
    constexpr int ROWB = kBlk * ELT;          // bytes per channel row of the tile
    constexpr int RMASK = FP8 ? 3 : 1;
    static_assert(NT >= THREADS, "one thread per (token quad, chunk) at least");
    const SeqView sv = seq_view(m, b, h);
    if (j * kBlk >= sv.n) return;  // the whole workgroup: past this sequence's end
    const int N = sv.n;
    const Strides st = m.st;
    const int64_t bh = int64_t(b) * m.H + h;
    const bool worker = NT == THREADS || int(threadIdx.x) < THREADS;
    const int q = threadIdx.x % (kBlk / 4), ch = threadIdx.x / (kBlk / 4), c0 = ch * 8;
    const uint16_t* base = v + sv.in_off;

    float inv[8];
    if constexpr (FP8) {
        if constexpr (FOLD) {
            if (threadIdx.x < DP) {
                const int nb = (N + kBlk - 1) / kBlk;
                const float* pp = vpart + sv.slot0 * DP + threadIdx.x;
                float a = 0.0f;
#pragma unroll 16
                for (int i = 0; i < nb; i++) a = fmaxf(a, pp[int64_t(i) * DP]);  // ascending blocks
                samax[threadIdx.x] = a;
            }
            __syncthreads();
        }
        auto amax_of = [&](int c) { return FOLD ? samax[c] : __uint_as_float(amax_bits[bh * DP + c]); };
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float a = worker ? amax_of(c0 + e) : 0.0f;
            inv[e] = a > 0.0f ? 448.0f / a : 0.0f;
        }
        if (j == 0 && threadIdx.x < DP) vscale[bh * DP + threadIdx.x] = amax_of(threadIdx.x) / 448.0f;
    }
    v8u16 r[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int t = j * kBlk + 4 * q + u;
        r[u] = v8u16{0, 0, 0, 0, 0, 0, 0, 0};
        if (worker && t < N && c0 < D) {
            const uint16_t* src = base + int64_t(t) * st.t + c0;
            if constexpr (VEC8) {
                r[u] = *(const v8u16*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) r[u][e] = (c0 + e < D) ? src[e] : (unsigned short)0;
            }
        }
    }
    if (worker) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int c = c0 + e;
            uint8_t* row = tile + (c ^ ((c >> 3) & RMASK)) * ROWB;
            float y[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const float x = in_to_f32<BF16>(r[u][e]);  // padding elements are +0
                y[u] = FP8 ? fminf(fmaxf(x * inv[e], -448.0f), 448.0f) : fminf(fmaxf(x, -65504.0f), 65504.0f);
            }
            if constexpr (FP8) {
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                *(int*)(row + 4 * q) = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
            } else {
                auto h2 = [&](int u) {
                    return uint32_t(f32_to_f16_bits(y[u])) | (uint32_t(f32_to_f16_bits(y[u + 1])) << 16);
                };
                *(uint2*)(row + 8 * q) = make_uint2(h2(0), h2(2));
            }
        }
    }
    __syncthreads();
    constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
    uint8_t* dst = (uint8_t*)vhat + (sv.slot0 + j) * int64_t(DP * ROWB);
    for (int i = threadIdx.x; i < DP * CPR; i += NT) {
        const int pr = i / CPR, k = i % CPR;
        const int c = pr ^ ((pr >> 3) & RMASK);
        *(uint4*)(dst + c * ROWB + 16 * k) = *(const uint4*)(tile + pr * ROWB + 16 * k);
    }
}

template <bool BF16, int DP, bool VEC8, bool FP8, bool FOLD = false>
__global__ __launch_bounds__(2 * DP) void quant_v_kernel(const uint16_t* __restrict__ v, SeqMap m, int D,
                                                      const uint32_t* __restrict__ amax_bits,
                                                      void* __restrict__ vhat, float* __restrict__ vscale,
                                                      const float* __restrict__ vpart = nullptr) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[DP * kBlk * (FP8 ? 1 : 2)];
    __shared__ float samax[FP8 && FOLD ? DP : 1];
    v_block<BF16, DP, VEC8, FP8, FOLD, 2 * DP>(v, m, D, amax_bits, vhat, vscale, vpart, blockIdx.x, blockIdx.y,
                                               blockIdx.z, tile, samax);
}

// Pass 1.  nq workgroups quantise four Q blocks each (number x of a (head, batch): x
// + nq4 * (h + Hq * b)); nkv take one K/V block each (j + NB * (h + H_kv * b)).  The
// two kinds are spread evenly over the grid, so Q's read-write stream and the K/V
// read streams run side by side.  VCAST (FP16 P.V, head dims up to 128): nkv more
// workgroups after those cast one V block each to the FP16 operand (quant_v_kernel's
// FP16 arithmetic, which needs no statistics), so no launch of its own is needed.
template <bool BF16, int DP, bool VEC8, bool VMAX, int QG, bool VCAST = false>
__global__ __launch_bounds__(256) void qkv_pass1_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, SeqMap mq, SeqMap mk, int D,
                                                        int nq, int nkv, int8_t* __restrict__ q_i8,
                                                        float* __restrict__ q_scale, double* __restrict__ kpart,
                                                        float* __restrict__ vpart, void* __restrict__ vhat = nullptr) {
    static_assert(!VCAST || (!VMAX && 2 * DP <= 256), "the V cast: FP16 mode, head dims up to 128");
    __shared__ __attribute__((aligned(16))) uint16_t tile[kBlk][DP];
    __shared__ float red[VMAX ? 256 / (DP / 8) : 1][DP];
    const int64_t wg = blockIdx.x, T = int64_t(nq) + nkv;
    if constexpr (VCAST) {
        if (wg >= T) {
            const int r = int(wg - T);
            const int j = r % mk.NB, h = (r / mk.NB) % mk.H, b = r / (mk.NB * mk.H);
            v_block<BF16, DP, VEC8, false, false, 256>(v, mk, D, nullptr, vhat, nullptr, nullptr, j, h, b,
                                                       (uint8_t*)&tile[0][0], nullptr);
            return;
        }
    }
    const int a0 = int(wg * nq / T), a1 = int((wg + 1) * nq / T);  // Q workgroups before wg, before wg + 1
    if (a1 > a0) {
        const int nq4 = (mq.NB + 3) / 4;
        const int x = a0 % nq4, h = (a0 / nq4) % mq.H, b = a0 / (nq4 * mq.H);
        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
        quant_block_wave<BF16, DP, VEC8, false, QG>(q, mq, D, nullptr, q_i8, q_scale, x * 4 + wave, h, b, lane);
    } else {
        const int r = int(wg) - a1;
        const int j = r % mk.NB, h = (r / mk.NB) % mk.H, b = r / (mk.NB * mk.H);
        kv_stats_block<BF16, DP, VEC8, VMAX>(k, v, mk, D, kpart, vpart, j, h, b, tile, red);
    }
}

// K operand of sage_quant_qkv for short sequences (at most kFoldBlocks blocks): each
// workgroup reduces its (b, kv head)'s K mean from the fp64 block sums of
// qkv_pass1_kernel itself, in qkv_pass2_kernel's order (ascending blocks), instead of a
// separate pass-2 launch; the x == 0 workgroup writes k_mean.  Then as
// quant_blocks_kernel.
constexpr int kFoldBlocks = 32;
template <bool BF16, int DP, bool VEC8, int G>
__global__ __launch_bounds__(256) void quant_k_fold_kernel(const uint16_t* __restrict__ k, SeqMap m, int D,
                                                           const double* __restrict__ kpart,
                                                           float* __restrict__ mean, int8_t* __restrict__ xq,
                                                           float* __restrict__ scale) {
    __shared__ float smean[DP];
    const int h = blockIdx.y, b = blockIdx.z, c = threadIdx.x;
    const SeqView sv = seq_view(m, b, h);
    if (c < D) {
        const int nb = (sv.n + kBlk - 1) / kBlk;
        const double* pp = kpart + sv.slot0 * D + c;
        double sum = 0.0;
#pragma unroll 16
        for (int i = 0; i < nb; i++) sum += pp[int64_t(i) * D];
        const float mu = sv.n > 0 ? float(sum / double(sv.n)) : 0.0f;
        smean[c] = mu;
        if (blockIdx.x == 0) mean[(int64_t(b) * m.H + h) * D + c] = mu;
    }
    __syncthreads();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    quant_block_wave<BF16, DP, VEC8, true, G, true>(k, m, D, smean, xq, scale, blockIdx.x * 4 + wave, h, b, lane);
}

// FP8 mode, head dims up to 128: the K codes and the V operand in one grid, once the K
// means and V maxima exist (after pass 2, or folded from pass 1's partials for short
// sequences).  Each (b, kv head) group has nb4 workgroups of four K blocks
// (quant_blocks_kernel / quant_k_fold_kernel) and NB of one V block (quant_v_kernel); the
// same arithmetic, one launch instead of two.  The groups run in descending order, the
// reverse of pass 1's, so that the K and V bytes pass 1 read last -- still held in part by
// the memory-side cache -- are read again first (3% less time at B4 H32 N8K D128 than the
// ascending order; the codes do not depend on the order).
template <bool BF16, int DP, bool VEC8, bool FOLD, int G>
__global__ __launch_bounds__(256) void kv_codes_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       SeqMap m, int D, int nk, const double* __restrict__ kpart,
                                                       float* __restrict__ mean, int8_t* __restrict__ xq,
                                                       float* __restrict__ scale, const uint32_t* __restrict__ amax_bits,
                                                       void* __restrict__ vhat, float* __restrict__ vscale,
                                                       const float* __restrict__ vpart) {
    static_assert(DP <= 128, "256 threads: one per (token quad, 8-channel chunk) of a V block");
    __shared__ float smean[FOLD ? DP : 1];
    __shared__ __attribute__((aligned(16))) uint8_t tile[DP * kBlk];
    __shared__ float samax[FOLD ? DP : 1];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nb4 = (m.NB + 3) / 4;
    // workgroup -> (group, K or V workgroup of the group): groups in descending order
    const int S = nb4 + m.NB;
    const int gi = nk / nb4 - 1 - int(blockIdx.x) / S, w = int(blockIdx.x) % S;  // nk = nb4 * H * B
    const int gh = gi % m.H, gb = gi / m.H;
    if (w < nb4) {
        const int x = nb4 - 1 - w, h = gh, b = gb;
        if constexpr (FOLD) {
            const SeqView sv = seq_view(m, b, h);
            const int c = threadIdx.x;
            if (c < D) {
                const int nb = (sv.n + kBlk - 1) / kBlk;
                const double* pp = kpart + sv.slot0 * D + c;
                double sum = 0.0;
#pragma unroll 16
                for (int i = 0; i < nb; i++) sum += pp[int64_t(i) * D];
                const float mu = sv.n > 0 ? float(sum / double(sv.n)) : 0.0f;
                smean[c] = mu;
                if (x == 0) mean[(int64_t(b) * m.H + h) * D + c] = mu;
            }
            __syncthreads();
            quant_block_wave<BF16, DP, VEC8, true, G, true>(k, m, D, smean, xq, scale, x * 4 + wave, h, b, lane);
        } else {
            quant_block_wave<BF16, DP, VEC8, true, G>(k, m, D, mean, xq, scale, x * 4 + wave, h, b, lane);
        }
    } else {
        const int j = m.NB - 1 - (w - nb4), h = gh, b = gb;
        v_block<BF16, DP, VEC8, true, FOLD, 256>(v, m, D, amax_bits, vhat, vscale, vpart, j, h, b, tile, samax);
    }
}

// ------------------------------------------------------------------------------------------
// Launchers
namespace {
template <bool BF16, int DP, bool VEC8>
hipError_t launch_qk_t(const QuantQKArgs& a, hipStream_t s) {
    const SeqMap mq = make_seq_map(a.layout_nhd, a.cu_q, a.B, a.Hq, a.Nq, a.total_q, a.D);
    const SeqMap mk = make_seq_map(a.layout_nhd, a.cu_k, a.B, a.Hkv, a.Nkv, a.total_k, a.D);
    k_mean_partial_kernel<BF16, DP, VEC8><<<dim3(mk.NB, a.Hkv, a.B), 256, 0, s>>>((const uint16_t*)a.k, mk, a.D,
                                                                                (double*)a.workspace);
    const int tot = a.B * a.Hkv * a.D;
    k_mean_final_kernel<<<(tot + 63) / 64, 64, 0, s>>>((const double*)a.workspace, mk, tot, a.D, a.k_mean);
    // K's codes right after its mean pass (the second read of K then finds part of it in
    // the memory-side cache), Q's after them
    quant_blocks_kernel<BF16, DP, VEC8, true><<<dim3((mk.NB + 3) / 4, a.Hkv, a.B), 256, 0, s>>>(
        (const uint16_t*)a.k, mk, a.D, a.k_mean, a.k_i8, a.k_scale);
    quant_blocks_kernel<BF16, DP, VEC8, false><<<dim3((mq.NB + 3) / 4, a.Hq, a.B), 256, 0, s>>>(
        (const uint16_t*)a.q, mq, a.D, nullptr, a.q_i8, a.q_scale);
    return hipGetLastError();
}

template <bool BF16, int DP, bool VEC8>
hipError_t launch_v_t(const QuantVArgs& a, hipStream_t s) {
    const SeqMap mv = make_seq_map(a.layout_nhd, a.cu_k, a.B, a.Hkv, a.Nkv, a.total_k, a.D);
    if (a.fp8) {
        const int n = a.B * a.Hkv * DP;
        uint32_t* amax = (uint32_t*)a.workspace;
        fill_zero_kernel<<<(n + 255) / 256, 256, 0, s>>>(amax, n);
        v_amax_kernel<BF16, DP, VEC8><<<dim3((mv.N + 255) / 256, a.Hkv, a.B), 256, 0, s>>>((const uint16_t*)a.v, mv,
                                                                                         a.D, amax);
        quant_v_kernel<BF16, DP, VEC8, true><<<dim3(mv.NB, a.Hkv, a.B), DP * 2, 0, s>>>(
            (const uint16_t*)a.v, mv, a.D, amax, a.v_hat, a.v_scale);
    } else {
        quant_v_kernel<BF16, DP, VEC8, false><<<dim3(mv.NB, a.Hkv, a.B), DP * 2, 0, s>>>(
            (const uint16_t*)a.v, mv, a.D, nullptr, a.v_hat, nullptr);
    }
    return hipGetLastError();
}

}  // namespace

template <bool BF16, int DP, bool VEC8, int QG, int KG>
hipError_t launch_qkv_t(const QuantQKArgs& a, const QuantVArgs& va, hipStream_t s) {
    const SeqMap mq = make_seq_map(a.layout_nhd, a.cu_q, a.B, a.Hq, a.Nq, a.total_q, a.D);
    const SeqMap mk = make_seq_map(a.layout_nhd, a.cu_k, a.B, a.Hkv, a.Nkv, a.total_k, a.D);
    const QKVWorkspace w = qkv_workspace(a.B, a.Hkv, a.Nkv, a.D, a.cu_k != nullptr, a.total_k, va.fp8);
    char* ws = (char*)a.workspace;
    double* kpart = (double*)(ws + w.kpart);
    float* vpart = (float*)(ws + w.vpart);
    uint32_t* amax = (uint32_t*)(ws + w.amax);
    const int nq = a.q != nullptr ? ((mq.NB + 3) / 4) * a.Hq * a.B : 0;  // sage_quant_kv: no Q
    const int nkv = mk.NB * a.Hkv * a.B;
    // head dims up to 128: FP16 P.V casts V in pass 1, FP8 P.V writes the K and V codes in
    // one launch (one launch fewer either way)
    constexpr bool kVCast = DP <= 128;
    if (mk.NB <= kFoldBlocks) {
        // short sequences: pass 2 folded into the K and V launches (three launches, two
        // at head dims up to 128)
        if (va.fp8)
            qkv_pass1_kernel<BF16, DP, VEC8, true, QG><<<nq + nkv, 256, 0, s>>>(
                (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)va.v, mq, mk, a.D, nq, nkv, a.q_i8,
                a.q_scale, kpart, vpart);
        else if constexpr (kVCast)
            qkv_pass1_kernel<BF16, DP, VEC8, false, QG, true><<<nq + 2 * nkv, 256, 0, s>>>(
                (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)va.v, mq, mk, a.D, nq, nkv, a.q_i8,
                a.q_scale, kpart, nullptr, va.v_hat);
        else
            qkv_pass1_kernel<BF16, DP, VEC8, false, QG><<<nq + nkv, 256, 0, s>>>(
                (const uint16_t*)a.q, (const uint16_t*)a.k, nullptr, mq, mk, a.D, nq, nkv, a.q_i8, a.q_scale, kpart,
                nullptr);
        if constexpr (kVCast) {
            if (va.fp8) {  // K and V codes in one launch
                const int nk = (mk.NB + 3) / 4 * a.Hkv * a.B;
                kv_codes_kernel<BF16, DP, VEC8, true, KG><<<nk + nkv, 256, 0, s>>>(
                    (const uint16_t*)a.k, (const uint16_t*)va.v, mk, a.D, nk, kpart, a.k_mean, a.k_i8, a.k_scale,
                    nullptr, va.v_hat, va.v_scale, vpart);
                return hipGetLastError();
            }
        }
        quant_k_fold_kernel<BF16, DP, VEC8, KG><<<dim3((mk.NB + 3) / 4, a.Hkv, a.B), 256, 0, s>>>(
            (const uint16_t*)a.k, mk, a.D, kpart, a.k_mean, a.k_i8, a.k_scale);
        if (va.fp8)
            quant_v_kernel<BF16, DP, VEC8, true, true><<<dim3(mk.NB, a.Hkv, a.B), DP * 2, 0, s>>>(
                (const uint16_t*)va.v, mk, a.D, nullptr, va.v_hat, va.v_scale, vpart);
        else if constexpr (!kVCast)
            quant_v_kernel<BF16, DP, VEC8, false><<<dim3(mk.NB, a.Hkv, a.B), DP * 2, 0, s>>>(
                (const uint16_t*)va.v, mk, a.D, nullptr, va.v_hat, nullptr);
        return hipGetLastError();
    }
    if (va.fp8) {
        qkv_pass1_kernel<BF16, DP, VEC8, true, QG><<<nq + nkv, 256, 0, s>>>(
            (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)va.v, mq, mk, a.D, nq, nkv, a.q_i8,
            a.q_scale, kpart, vpart);
        qkv_pass2_kernel<DP, true><<<(a.B * a.Hkv * DP + 63) / 64, 64, 0, s>>>(kpart, vpart, mk, a.B, a.D, a.k_mean,
                                                                             amax);
    } else {
        if constexpr (kVCast)
            qkv_pass1_kernel<BF16, DP, VEC8, false, QG, true><<<nq + 2 * nkv, 256, 0, s>>>(
                (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)va.v, mq, mk, a.D, nq, nkv, a.q_i8,
                a.q_scale, kpart, nullptr, va.v_hat);
        else
            qkv_pass1_kernel<BF16, DP, VEC8, false, QG><<<nq + nkv, 256, 0, s>>>(
                (const uint16_t*)a.q, (const uint16_t*)a.k, nullptr, mq, mk, a.D, nq, nkv, a.q_i8, a.q_scale, kpart,
                nullptr);
        qkv_pass2_kernel<DP, false><<<(a.B * a.Hkv * DP + 63) / 64, 64, 0, s>>>(kpart, nullptr, mk, a.B, a.D,
                                                                              a.k_mean, nullptr);
    }
    if constexpr (kVCast) {
        if (va.fp8) {  // K and V codes in one launch
            const int nk = (mk.NB + 3) / 4 * a.Hkv * a.B;
            kv_codes_kernel<BF16, DP, VEC8, false, KG><<<nk + nkv, 256, 0, s>>>(
                (const uint16_t*)a.k, (const uint16_t*)va.v, mk, a.D, nk, nullptr, a.k_mean, a.k_i8, a.k_scale, amax,
                va.v_hat, va.v_scale, nullptr);
            return hipGetLastError();
        }
    }
    quant_blocks_kernel<BF16, DP, VEC8, true, KG><<<dim3((mk.NB + 3) / 4, a.Hkv, a.B), 256, 0, s>>>(
        (const uint16_t*)a.k, mk, a.D, a.k_mean, a.k_i8, a.k_scale);
    if (va.fp8)
        quant_v_kernel<BF16, DP, VEC8, true><<<dim3(mk.NB, a.Hkv, a.B), DP * 2, 0, s>>>(
            (const uint16_t*)va.v, mk, a.D, amax, va.v_hat, va.v_scale);
    else if constexpr (!kVCast)
        quant_v_kernel<BF16, DP, VEC8, false><<<dim3(mk.NB, a.Hkv, a.B), DP * 2, 0, s>>>(
            (const uint16_t*)va.v, mk, a.D, nullptr, va.v_hat, nullptr);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_qk_dp(const QuantQKArgs& a, hipStream_t s) {
    const bool vec = (a.D % 8) == 0;
    if (a.D <= 64) return vec ? launch_qk_t<BF16, 64, true>(a, s) : launch_qk_t<BF16, 64, false>(a, s);
    if (a.D <= 128) return vec ? launch_qk_t<BF16, 128, true>(a, s) : launch_qk_t<BF16, 128, false>(a, s);
    return vec ? launch_qk_t<BF16, 256, true>(a, s) : launch_qk_t<BF16, 256, false>(a, s);
}

hipError_t launch_quant_qk(const QuantQKArgs& a, hipStream_t s) {
    return a.bf16 ? launch_qk_dp<true>(a, s) : launch_qk_dp<false>(a, s);
}

template <bool BF16>
hipError_t launch_v_dp(const QuantVArgs& a, hipStream_t s) {
    const bool vec = (a.D % 8) == 0;
    if (a.D <= 64) return vec ? launch_v_t<BF16, 64, true>(a, s) : launch_v_t<BF16, 64, false>(a, s);
    if (a.D <= 128) return vec ? launch_v_t<BF16, 128, true>(a, s) : launch_v_t<BF16, 128, false>(a, s);
    return vec ? launch_v_t<BF16, 256, true>(a, s) : launch_v_t<BF16, 256, false>(a, s);
}

hipError_t launch_quant_v(const QuantVArgs& a, hipStream_t s) {
    return a.bf16 ? launch_v_dp<true>(a, s) : launch_v_dp<false>(a, s);
}

template <bool BF16, int QG, int KG>
hipError_t launch_qkv_g(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t s) {
    const bool vec = (a.D % 8) == 0;
    if (a.D <= 64)
        return vec ? launch_qkv_t<BF16, 64, true, QG, KG>(a, v, s) : launch_qkv_t<BF16, 64, false, QG, KG>(a, v, s);
    if (a.D <= 128)
        return vec ? launch_qkv_t<BF16, 128, true, QG, KG>(a, v, s) : launch_qkv_t<BF16, 128, false, QG, KG>(a, v, s);
    return vec ? launch_qkv_t<BF16, 256, true, QG, KG>(a, v, s) : launch_qkv_t<BF16, 256, false, QG, KG>(a, v, s);
}
template <bool BF16>
hipError_t launch_qkv_dp(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t s) {
    // per-thread granularity: one Q scale per token, one K scale per 32 keys
    return a.thread_gran ? launch_qkv_g<BF16, 1, 32>(a, v, s) : launch_qkv_g<BF16, 64, 64>(a, v, s);
}

hipError_t launch_quant_qkv(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t s) {
    return a.bf16 ? launch_qkv_dp<true>(a, v, s) : launch_qkv_dp<false>(a, v, s);
}

// ---- the fused quantisation's workspace in static device memory --------------------
// For callers that cannot allocate (sage_quant_qkv_noalloc).  Every device the library
// runs on holds one copy for the life of the process.  In host code the array's name
// stands for a host-side shadow, not for the device copy, so kernels only ever receive
// the device address that hipGetSymbolAddress reports, fetched once per device (with
// that device current) on its first use.  The fused launch sequence writes every part
// of the workspace it reads, so nothing in it has to start at zero.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<uintptr_t> g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void* d = nullptr;
        e = hipGetSymbolAddress(&d, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (d == nullptr) return hipErrorInvalidSymbol;
        p = reinterpret_cast<uintptr_t>(d);
        g_scratch_ptr[dev].store(p, std::memory_order_release);  // same value if two threads race here
    }
    *ptr = reinterpret_cast<void*>(p);
    return hipSuccess;
}


// ------------------------------------------------------------------------------------------
// Microscaling FP4 (the README's "SageAttention3: Microscaling FP4 Attention", taken as
// the OCP MX v1.0 MXFP4 format that gfx950's scaled matrix instructions read): every
// 32 consecutive elements along a contraction axis share the power-of-two scale
// X = 2^E, E = floor(log2 amax) - 2 held to [-126, 127] (an all-zero block: -126),
// stored as the E8M0 byte E + 127; elements are e2m1(x / X), round to nearest even,
// saturating at 6, as 4-bit codes (element 2t in the low nibble of byte t).
//   Q, smoothed K: per token, blocks of 32 channels -> codes [row][Dp/2], exponents
//                  [row][Dp/32] (rows and block slots as for INT8);
//   V:             per channel, blocks of 32 tokens; per 64-token slot the codes
//                  [Dp][32] (channel-major) and the exponents in the order
//                  [token half g][channel % 32][channel / 32], so that the lane of the
//                  P.V matrix instruction holding channel 32 t + i, half g finds its
//                  Dp / 32 exponents in one word.

__device__ __forceinline__ int mx_exp(float amax) {  // amax >= 0 (a zero or subnormal amax gives -126)
    return max(int((__float_as_uint(amax) >> 23) & 0xffu) - 129, -126);
}
__device__ __forceinline__ float mx_scale_f32(int E) { return __uint_as_float(uint32_t(E + 127) << 23); }

// Q or K: one wave per 64-token block; lane l covers 8 channels (chunk l % CH) of the
// token rows l / CH + p * (64 / CH); the four lanes of a 32-channel block (aligned
// groups of four lanes) combine their maxima with two lane exchanges.
template <bool BF16, int DP, bool VEC8, bool SMOOTH>
__global__ __launch_bounds__(256) void mx_rows_kernel(const uint16_t* __restrict__ x, SeqMap m, int D,
                                                      const float* __restrict__ mean, uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xe) {
    constexpr int CH = DP / 8, RPP = kWave / CH, PASSES = kBlk / RPP;
    const int lane = threadIdx.x % kWave;
    // smoothed K follows the mean pass, which read K in ascending order: descending here,
    // so the blocks read last (still partly in the memory-side cache) come first
    const int bx = SMOOTH ? int(gridDim.x - 1 - blockIdx.x) : int(blockIdx.x);
    const int j = bx * 4 + int(threadIdx.x / kWave);
    const int h = SMOOTH ? int(gridDim.y - 1 - blockIdx.y) : int(blockIdx.y);
    const int b = SMOOTH ? int(gridDim.z - 1 - blockIdx.z) : int(blockIdx.z);
    const SeqView sv = seq_view(m, b, h);
    if (j * kBlk >= sv.n) return;  // this wave: past the sequence's end
    const int N = sv.n;
    const Strides st = m.st;
    const int64_t bh = int64_t(b) * m.H + h;
    const int ch = lane % CH, r0 = lane / CH, c0 = ch * 8;
    const uint16_t* base = x + sv.in_off;
    float mu[8];
#pragma unroll
    for (int e = 0; e < 8; e++) mu[e] = (SMOOTH && c0 + e < D) ? mean[bh * D + c0 + e] : 0.0f;
#pragma unroll 4
    for (int p = 0; p < PASSES; p++) {
        const int t = j * kBlk + p * RPP + r0;
        v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < N && c0 < D) {
            const uint16_t* src = base + int64_t(t) * st.t + c0;
            if constexpr (VEC8) {
                r = *(const v8u16*)src;
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) r[e] = (c0 + e < D) ? src[e] : (unsigned short)0;
            }
        }
        float y[8], am = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const bool real = t < N && c0 + e < D;  // padding tokens and channels: +0
            y[e] = real ? in_to_f32<BF16>(r[e]) - mu[e] : 0.0f;
            am = fmaxf(am, fabsf(y[e]));
        }
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        const int E = mx_exp(am);
        const float X = mx_scale_f32(E);
        int w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], X, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], X, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], X, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], X, 3);
        const int64_t row = sv.row0 + t;
        *(int*)(xq + row * (DP / 2) + 4 * ch) = w;
        if ((ch & 3) == 0) xe[row * (DP / 32) + ch / 4] = uint8_t(E + 127);
    }
}

// V: one workgroup of 2 Dp threads per 64-token block; the block's 64 x Dp tile is
// read with 16-byte loads into LDS, then thread 2 d + g quantises channel d over the
// tokens 32 g .. 32 g + 31 and writes its 16 code bytes (consecutive threads,
// consecutive bytes) and its exponent.
template <bool BF16, int DP, bool VEC8>
__global__ __launch_bounds__(2 * DP) void mx_v_kernel(const uint16_t* __restrict__ v, SeqMap m, int D,
                                                      uint8_t* __restrict__ vq, uint8_t* __restrict__ ve) {
    constexpr int CH = DP / 8, THREADS = 2 * DP, RPP = THREADS / CH;  // RPP token rows per pass
    constexpr int LD = DP + 8;                                        // LDS row pitch (elements)
    __shared__ __attribute__((aligned(16))) uint16_t tile[kBlk * LD];
    const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const SeqView sv = seq_view(m, b, h);
    if (j * kBlk >= sv.n) return;  // the whole workgroup: past this sequence's end
    const int N = sv.n;
    const Strides st = m.st;
    const uint16_t* base = v + sv.in_off;
    {
        const int ch = threadIdx.x % CH, r0 = threadIdx.x / CH, c0 = ch * 8;
#pragma unroll
        for (int p = 0; p < kBlk / RPP; p++) {
            const int tl = p * RPP + r0, t = j * kBlk + tl;
            v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
            if (t < N && c0 < D) {
                const uint16_t* src = base + int64_t(t) * st.t + c0;
                if constexpr (VEC8) {
                    r = *(const v8u16*)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++) r[e] = (c0 + e < D) ? src[e] : (unsigned short)0;
                }
            }
            *(v8u16*)&tile[tl * LD + c0] = r;
        }
    }
    __syncthreads();
    const int d = threadIdx.x >> 1, g = threadIdx.x & 1;
    float y[32], am = 0.0f;
#pragma unroll
    for (int u = 0; u < 32; u++) {
        y[u] = in_to_f32<BF16>(tile[(32 * g + u) * LD + d]);  // padding: +0
        am = fmaxf(am, fabsf(y[u]));
    }
    const int E = mx_exp(am);
    const float X = mx_scale_f32(E);
    int w[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        int x = 0;
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * k + 0], y[8 * k + 1], X, 0);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * k + 2], y[8 * k + 3], X, 1);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * k + 4], y[8 * k + 5], X, 2);
        x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * k + 6], y[8 * k + 7], X, 3);
        w[k] = x;
    }
    const int64_t slot = sv.slot0 + j;
    *(int4*)(vq + (slot * DP + d) * 32 + 16 * g) = make_int4(w[0], w[1], w[2], w[3]);
    ve[slot * DP * 2 + (g * 32 + (d & 31)) * (DP / 32) + (d >> 5)] = uint8_t(E + 127);
}

namespace {
template <bool BF16, int DP, bool VEC8>
hipError_t launch_mx_t(const QuantMXArgs& a, hipStream_t s) {
    const SeqMap mq = make_seq_map(a.layout_nhd, a.cu_q, a.B, a.Hq, a.Nq, a.total_q, a.D);
    const SeqMap mk = make_seq_map(a.layout_nhd, a.cu_k, a.B, a.Hkv, a.Nkv, a.total_k, a.D);
    k_mean_partial_kernel<BF16, DP, VEC8><<<dim3(mk.NB, a.Hkv, a.B), 256, 0, s>>>((const uint16_t*)a.k, mk, a.D,
                                                                                (double*)a.workspace);
    const int tot = a.B * a.Hkv * a.D;
    k_mean_final_kernel<<<(tot + 63) / 64, 64, 0, s>>>((const double*)a.workspace, mk, tot, a.D, a.k_mean);
    // K's codes right after its mean pass (the second read of K then finds part of it in
    // the memory-side cache), then Q's
    mx_rows_kernel<BF16, DP, VEC8, true><<<dim3((mk.NB + 3) / 4, a.Hkv, a.B), 256, 0, s>>>(
        (const uint16_t*)a.k, mk, a.D, a.k_mean, a.k4, a.k4_exp);
    if (a.q != nullptr)  // sage_quant_mxfp4_kv: no Q
        mx_rows_kernel<BF16, DP, VEC8, false><<<dim3((mq.NB + 3) / 4, a.Hq, a.B), 256, 0, s>>>(
            (const uint16_t*)a.q, mq, a.D, nullptr, a.q4, a.q4_exp);
    mx_v_kernel<BF16, DP, VEC8><<<dim3(mk.NB, a.Hkv, a.B), 2 * DP, 0, s>>>((const uint16_t*)a.v, mk, a.D, a.v4,
                                                                          a.v4_exp);
    return hipGetLastError();
}
template <bool BF16>
hipError_t launch_mx_dp(const QuantMXArgs& a, hipStream_t s) {
    const bool vec = (a.D % 8) == 0;
    if (a.D <= 64) return vec ? launch_mx_t<BF16, 64, true>(a, s) : launch_mx_t<BF16, 64, false>(a, s);
    if (a.D <= 128) return vec ? launch_mx_t<BF16, 128, true>(a, s) : launch_mx_t<BF16, 128, false>(a, s);
    return vec ? launch_mx_t<BF16, 256, true>(a, s) : launch_mx_t<BF16, 256, false>(a, s);
}
}  // namespace

hipError_t launch_quant_mxfp4(const QuantMXArgs& a, hipStream_t s) {
    return a.bf16 ? launch_mx_dp<true>(a, s) : launch_mx_dp<false>(a, s);
}

}  // namespace sage
