// attn_fwd.hip -- fused INT8-QK / FP16-or-FP8-PV attention forward for gfx950.
//
// Method (SageAttention project README, "Current Features" and "Available APIs";
// trdm.cn 9070XT blog, section 2.2): scores S32 = Q^ K^T come from INT8 x INT8 -> INT32
// matrix-core products, are dequantised with the per-64-token block scales of Q and
// K, and feed an online base-2 softmax (running row max m, running row sum l); P is
// rounded to FP16 or FP8-e4m3 and multiplied with V^ on the matrix cores with fp32
// accumulation.  The README's two-level accumulation (short sums in a reduced-precision
// tensor-core accumulator, added into fp32) guards against an inner accumulator that
// gfx950 does not have: its FP8/FP16 matrix instructions add their products straight
// into an fp32 operand.  The two-level mode name therefore runs the single-level fp32
// accumulation; the literal form (a fresh fp32 partial per tile plus a vector add) is
// kept as its own mode (pv_tile's TL) and rounds the accumulator slightly differently.
//
// gfx950 design:
//  * workgroup = 4 waves = 128 queries; each wave owns 32 queries inside one 64-token Q
//    block (wave-uniform Q scale) and walks 64-key tiles (one K block: uniform K scale);
//  * the vector ALU, not the matrix core, bounds this kernel: per score the softmax
//    issues about five vector instructions, two of them (exp2, the FP8 pack) at a
//    quarter of the full rate, against about half as many cycles of MFMA.  A wave on
//    its own issues vector instructions at about a quarter of the rate the ALU
//    sustains with four ready waves, so the schedule is kept simple and small (no
//    score double buffer: 164 VGPRs at head dim 128) to fit three waves per SIMD (four
//    at head dim 64), which keep the ALU fed while others wait on the matrix core,
//    LDS or the barrier;
//  * K^ and V^ tiles stream HBM -> LDS with direct-to-LDS 16-byte loads, two tiles
//    ahead (three LDS stages; one ahead for FP16 P.V at head dim 128, whose 24 KB
//    stages fit only twice per workgroup), the same number of loads per thread per tile (so
//    explicit vmcnt waits are exact), XOR-swizzled so every 16-byte operand read is
//    bank-conflict free;
//  * S^T = K^ Q^T on v_mfma_i32_32x32x32_i8 (keys on the M side): each lane holds one
//    query column, so row max / row sum are lane-local plus one exchange between the
//    two lane halves; at head dims up to 128 the accumulators start at the bits of
//    fp32 1/(2 pi), so each INT32 result read as fp32 is 1/(2 pi) + S32 * 2^-26 exactly
//    and the softmax needs no integer-to-float conversion (5-10% faster);
//  * the K^ rows fed to each MFMA row are permuted so that the INT32 result lands in
//    exactly the register order the P.V MFMA wants for its B operand: P never leaves
//    registers; V^ tiles are stored channel-major so the A operand is contiguous;
//  * P.V on v_mfma_scale_f32_32x32x64_f8f6f4 (FP8, unit scales) or
//    v_mfma_f32_32x32x16_f16 (FP16), output O^T accumulated in fp32 registers;
//  * consecutive workgroups on one XCD take the query tiles of one (b, kv head), so
//    the K^/V^ tiles they all stream come from that XCD's L2 (causal: heaviest tiles
//    of the head first, for load balance).
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace sage {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Score offset: the accumulators of the score instructions start at the bits of the
// inline constant 1/(2 pi) (0x3E22F983), so the INT32 result C + s read as fp32 is
// 1/(2 pi) + s * 2^-26 exactly for -2292099 <= s <= 6096508 (one binade) -- every score
// at head dims up to 128 (|s| <= 128 * 127^2) -- and no conversion is needed.
constexpr int kScoreBias = 0x3E22F983;
// log2(448) = 8.8073549..., rounded down by ~1e-6 so that 2^(t + c) stays below 448
// for t <= 0 even with a one-ulp exp2 error: FP8 P is produced directly as p * 448
// (the e4m3 maximum), with a relative bias of about 6e-7.
constexpr float kLog2_448 = 8.807354f;
// FP16 P.V: how far (log2 units) the running maximum may rise above the reference
// maximum before the accumulators are rescaled
constexpr float kLazyLog2 = 8.0f;


// Mode constants.  DP = padded head dim (64 | 128 | 256); FP8 = P.V in e4m3 (else fp16).
template <int DP, bool FP8>
struct Cfg {
    static constexpr int WAVES = 4;  // one wave per SIMD; OCC workgroups share a CU
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int QW = 32;            // queries per wave
    static constexpr int BM = WAVES * QW;    // queries per workgroup
    static constexpr int VELT = FP8 ? 1 : 2;
    static constexpr int KROW = DP;          // bytes per K^ row (one key)
    static constexpr int VROW = kBlk * VELT; // bytes per V^ row (one channel of 64 keys)
    static constexpr int KBYTES = kBlk * KROW;
    static constexpr int VBYTES = DP * VROW;
    static constexpr int KCHUNKS = KBYTES / 16;
    static constexpr int VCHUNKS = VBYTES / 16;
    // every thread issues ROUNDS 16-byte loads per tile: KROUNDS for K^, then V^
    static constexpr int KROUNDS = KCHUNKS / THREADS;
    static constexpr int ROUNDS = (KCHUNKS + VCHUNKS) / THREADS;
    static constexpr int STAGE = ROUNDS * THREADS * 16;
    static_assert(KCHUNKS % THREADS == 0 && VCHUNKS % THREADS == 0, "each load round lies in one region");
    // Per wave, QK^T, softmax, rescale and P.V of a tile run in turn, with no score
    // double buffer, so a wave fits in 168 VGPRs (128 at head dim 64) and three (four)
    // waves share each SIMD.  The vector ALU is the binding unit -- the softmax costs
    // about twice the MFMA time -- and one wave can issue a vector instruction only
    // every other slot, so the ALU needs several ready waves per SIMD to stay busy.
    // (head dim 256: 128 accumulator VGPRs alone, two waves; one with FP16 P.V, whose
    // operand registers take it past 256 VGPRs)
    static constexpr int OCC = DP == 64 ? 4 : (DP == 128 ? 3 : (FP8 ? 2 : 1));  // waves per SIMD
    // LDS stages: three (two tiles stream in while one is used) when OCC workgroups of
    // three fit in the 160 KB of a CU, else two
    static constexpr int NST = OCC * 3 * STAGE <= 160 * 1024 ? 3 : 2;
    static constexpr int KS = DP / 32;  // MFMA k-steps of QK^T
    static constexpr int DT = DP / 32;  // 32-channel tiles of O^T
    // XOR swizzles: bit c of the chunk flip is parity(row & mask_c); each is
    // conflict-free for the operand reads below with 8 lanes x 128 B or 16 lanes x
    // 256 B served per LDS cycle.
    static constexpr uint32_t KM0 = DP == 128 ? 0x2u : 0x6u;
    static constexpr uint32_t KM1 = DP == 128 ? 0x5u : (FP8 ? 0x20u : 0x8u);
    static constexpr uint32_t KM2 = DP == 128 ? (FP8 ? 0x20u : 0x8u) : 0x0u;
    static constexpr uint32_t VM0 = FP8 ? 0x4u : 0x2u;
    static constexpr uint32_t VM1 = FP8 ? 0xAu : 0x4u;
    static constexpr uint32_t VM2 = FP8 ? 0x0u : 0x9u;
};

template <class C>
__device__ __forceinline__ int kswz(int row) {
    if constexpr (C::KROW == 256) {
        // 16 chunks per row and every row on the same banks: the 16 lanes served per
        // LDS cycle read 16 different rows (bits 0-2 and 5 of the row for FP8's key
        // order, bits 0-3 for FP16's), which this XOR maps onto 16 distinct chunks
        return C::VELT == 1 ? ((row & 7) | (((row >> 5) & 1) << 3)) : (row & 15);
    } else {
        return parity(row & C::KM0) | (parity(row & C::KM1) << 1) | (parity(row & C::KM2) << 2);
    }
}
template <class C>
__device__ __forceinline__ int vswz(int row) {
    return parity(row & C::VM0) | (parity(row & C::VM1) << 1) | (parity(row & C::VM2) << 2);
}

// Key (0..63 within a tile) whose K^ row feeds row i (0..31) of QK^T MFMA tile kt.
// Chosen so that the C-layout of the result (lane half g, register r) equals the
// B-operand layout of the P.V MFMA over keys:
//   FP8:  lane half g holds keys 32g .. 32g+31 (tile kt: +16kt + r);
//   FP16: MFMA m (16 keys) takes keys 16m + 8g + e from tile m/2, registers 8(m%2)+e.
template <bool FP8>
__device__ __forceinline__ int key_of_row(int kt, int i) {
    const int a = i >> 3, g = (i >> 2) & 1, b = i & 3;
    if constexpr (FP8) return 32 * g + 16 * kt + 4 * a + b;
    else return 32 * kt + 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}
// Key held by lane half g, register r of result tile kt (C layout row 8(r/4)+4g+r%4).
template <bool FP8>
__device__ __forceinline__ int key_of_reg(int kt, int g, int r) {
    return key_of_row<FP8>(kt, 8 * (r >> 2) + 4 * g + (r & 3));
}

// Per-thread source offsets of the direct-to-LDS loads, computed once: round u of
// every thread covers LDS chunk u * THREADS + tid, which lies wholly in the K^ region
// (rounds < KROUNDS) or the V^ region, so each round has a single uniform base.
template <class C>
struct DmaPlan {
    uint32_t off[C::ROUNDS];
};
template <class C>
__device__ __forceinline__ DmaPlan<C> make_dma_plan(int tid) {
    DmaPlan<C> d;
#pragma unroll
    for (int u = 0; u < C::ROUNDS; u++) {
        const int ci = u * C::THREADS + tid;
        if (u < C::KROUNDS) {
            const int row = ci / (C::KROW / 16), cpos = ci % (C::KROW / 16);
            d.off[u] = uint32_t(row * C::KROW + 16 * (cpos ^ kswz<C>(row)));
        } else {
            const int vi = ci - C::KCHUNKS;
            const int row = vi / (C::VROW / 16), cpos = vi % (C::VROW / 16);
            d.off[u] = uint32_t(row * C::VROW + 16 * (cpos ^ vswz<C>(row)));
        }
    }
    return d;
}
// lds_wave_base: LDS byte address of the stage plus this wave's 1 KB slot of round 0;
// rounds U .. END-1 (END = KROUNDS: the K^ region alone)
template <class C, int U = 0, int END = C::ROUNDS>
__device__ __forceinline__ void issue_stage(uint32_t lds_wave_base, const int8_t* ktile, const uint8_t* vtile,
                                            const DmaPlan<C>& d) {
    if constexpr (U < END) {
        const void* base = U < C::KROUNDS ? (const void*)ktile : (const void*)vtile;
        load_lds_16_s<U * C::THREADS * 16>(base, d.off[U], lds_wave_base);
        issue_stage<C, U + 1, END>(lds_wave_base, ktile, vtile, d);
    }
}

// S^T tiles of one 64-key tile for this wave's 32 queries: S[kt] (keys through the
// permutation above on M, queries lane%32 on N).
template <class C, bool FP8, bool OFS = false>
__device__ __forceinline__ void qk_tile(const uint8_t* __restrict__ kst, const v4i (&qf)[C::KS], v16i (&S)[2],
                                        int lane) {
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        const int row = key_of_row<FP8>(kt, i);
        const int sw = kswz<C>(row);
        const uint8_t* rbase = kst + row * C::KROW;
#pragma unroll
        for (int s = 0; s < C::KS; s++) {
            const v4i a = lds_read_16(rbase + 16 * ((2 * s + g) ^ sw));
            if (s == 0) {
                constexpr int b = OFS ? kScoreBias : 0;
                const v16i z = {b, b, b, b, b, b, b, b, b, b, b, b, b, b, b, b};
                S[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], z, 0, 0, 0);
            } else {
                S[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[s], S[kt], 0, 0, 0);
            }
        }
    }
}

template <class C>
__device__ __forceinline__ void load_q_frags(v4i (&qf)[C::KS], const int8_t* qrows, int lane) {
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int s = 0; s < C::KS; s++) qf[s] = *(const v4i*)(qrows + i * C::KROW + 32 * s + 16 * g);
}

// P in the B-operand registers of the P.V MFMAs: FP8 e4m3 codes of p * 448 (one
// 64-key MFMA), or fp16 (four 16-key MFMAs).
template <bool FP8>
struct PPack;
template <>
struct PPack<true> {
    v8i b;
};
template <>
struct PPack<false> {
    v8h b[4];
};

// Online softmax step for one tile: updates m, l, returns alpha and writes P straight
// into the P.V operand registers (FP8: e4m3 of p * 448; FP16: fp16 of p), four values
// at a time, so no array of fp32 probabilities is ever live.  Masked keys get INT32_MIN
// and p = 0.  m is the reference maximum: with FP8 P the running max fp32(S32max c), the
// scheme's fp32 score maximum; with FP16 P the running max as it stood when it last rose
// by more than kLazyLog2 (below).  t = S32 c - m is formed with one rounding (fma) from
// the exact score, so with FP8 P, p differs from
// the two-rounding fp32 evaluation fp32(2^fp32(fp32(S32 c) - m)) by at most half an ulp
// of the score (plus half an ulp of m - log2 448 with FP8), a few 1e-5 relative at
// |S2| < 2^10.  OFS (offset scores, head dims up to 128): S holds the bits of K0 + S32
// 2^-26, so the row max is taken on those bits (same order) and value - K0 = S32 2^-26
// exactly (one binade), which times c 2^26 is S32 c: the score needs one subtraction
// of an inline constant instead of an integer-to-float conversion.
// kmax: the last key this lane's query may see when causal.
// c0, c1: dequantisation factors of score tiles 0 and 1 (equal unless K carries one
// scale per 32 keys with FP16 P.V, whose tile kt holds keys 32 kt .. 32 kt + 31).
template <bool FP8, bool MASK, bool CAUSAL, bool C2 = false, bool OFS = false>
__device__ __forceinline__ float softmax_tile(v16i (&S)[2], PPack<FP8>& pk, float c0, float c1, float& m, float& l,
                                              int g, int key0, int kmax, int Nkv) {
    int tvis = 0;  // MASK: register r of tile kt is visible iff key_of_reg(kt, 0, r) < tvis
    if constexpr (MASK) {
        // key key0 + key_of_reg(kt, g, r) is visible iff it is below min(Nkv, kmax + 1)
        // (causal) or Nkv; key_of_reg(kt, g, r) = key_of_reg(kt, 0, r) + (32 | 8) * g,
        // so one per-lane threshold against compile-time offsets decides every
        // register.  The threshold is kept opaque: otherwise the compiler proves it
        // loop-invariant on the tail tile and hoists 32 masks out of the tile loop.
        int lim = Nkv;
        if constexpr (CAUSAL) lim = min(lim, kmax + 1);
        int t = lim - key0 - (FP8 ? 32 : 8) * g;
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (!(key_of_reg<FP8>(kt, 0, r) < t)) S[kt][r] = INT32_MIN;
        tvis = t;
    }
    // row max: two chains of three-input maxima (v_max3), one per score tile
    int mxk[2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        int a = max(max(S[kt][0], S[kt][1]), S[kt][2]);
#pragma unroll
        for (int r = 3; r + 1 < 16; r += 2) a = max(max(a, S[kt][r]), S[kt][r + 1]);
        mxk[kt] = max(a, S[kt][15]);
    }
    // OFS: the offset scores' float values are K0 + s 2^-26, so (value - K0) = s 2^-26
    // exactly (same binade) and times c 2^26 gives fp32(s c), as float(s) * c would
    const float K0 = __int_as_float(kScoreBias);
    const float c0s = OFS ? c0 * 67108864.0f : c0, c1s = OFS ? c1 * 67108864.0f : c1;
    auto sf = [&](int x) { return OFS ? __int_as_float(x) - K0 : float(x); };
    float tmax;
    if constexpr (C2) {
        // each tile's maximum with its own factor (float(S) * c is monotone in S)
        const float t0 = (MASK && mxk[0] == INT32_MIN) ? -1e30f : sf(mxk[0]) * c0s;
        const float t1 = (MASK && mxk[1] == INT32_MIN) ? -1e30f : sf(mxk[1]) * c1s;
        tmax = fmaxf(t0, t1);
    } else {
        const int mx = max(mxk[0], mxk[1]);
        tmax = (MASK && mx == INT32_MIN) ? -1e30f : sf(mx) * c0s;
    }
    tmax = halves_max(tmax);
    float mnew = fmaxf(m, tmax);
    // FP16 P: the reference maximum moves only when the tile's maximum exceeds it by more
    // than kLazyLog2 (so p <= 2^kLazyLog2, far inside fp16's range, and the 64-accumulator
    // rescale runs a few times per row instead of whenever the maximum creeps up).  P is
    // then fp16(2^(S c - m)) against a reference up to kLazyLog2 below the running maximum:
    // the same softmax, with fp16's relative rounding of p unchanged.  FP8 P must stay
    // <= 1 (448 p <= 448), so FP8 keeps the running maximum itself.
    if constexpr (!FP8) mnew = mnew > m + kLazyLog2 ? mnew : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    float negm = FP8 ? kLog2_448 - mnew : -mnew;
    if constexpr (FP8) {
        // 448 p of the maximum exceeds 448 by at most the roundings of m and of negm
        // (1.5 ulp of m: 2^-11 relative at |m| < 2^12, far inside the [448, 464) that
        // e4m3's round-to-nearest maps to 448); from |m| = 2^12 on the bias backs off by
        // 8 ulps of m, so that 2^(t + log2 448) stays at or below 448 by construction
        negm = fabsf(mnew) >= 4096.0f ? __builtin_fmaf(fabsf(mnew), -0x1p-20f, negm) : negm;
    }
    float acc[4];
#pragma unroll
    for (int w = 0; w < 8; w++) {
        const int kt = w >> 2, r0 = 4 * (w & 3);
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            q[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sf(S[kt][r0 + e]), kt ? c1s : c0s, negm));
            // the same predicate as above (compiled to a scalar-mask select, not VCC)
            if constexpr (MASK) q[e] = key_of_reg<FP8>(kt, 0, r0 + e) < tvis ? q[e] : 0.0f;
            acc[e] = w == 0 ? q[e] : acc[e] + q[e];
        }
        if constexpr (FP8) {
            // the low half is written first; the register's previous contents are don't-care,
            // so it reuses q[1]'s (dead after this point) instead of a zeroed one
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], __float_as_int(q[1]), false);
            pk.b[w] = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++) pk.b[2 * kt + (r0 >> 3)][(r0 & 7) + e] = (_Float16)q[e];
        }
    }
    l = __builtin_fmaf(l, alpha, (acc[0] + acc[1]) + (acc[2] + acc[3]));
    return alpha;
}

// O^T += V^T P^T for one tile; vst = the V^ region of the tile's LDS stage.
// TL = false: the products accumulate straight into O (the matrix instruction adds its
// sum to the fp32 accumulator operand).  TL = true: the explicit two-level form of the
// README's two-level accumulation -- each tile's products go into a fresh fp32 partial,
// which one vector add then folds into O.
template <class C, bool FP8, bool TL = false>
__device__ __forceinline__ void pv_tile(const uint8_t* __restrict__ vst, const PPack<FP8>& pk, v16f (&O)[C::DT],
                                        int lane) {
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++) {
        const int d = 32 * dt + i;
        const int sw = vswz<C>(d);
        const uint8_t* rb = vst + d * C::VROW;
        v16f acc = TL ? v16f{} : O[dt];
        if constexpr (FP8) {
            const v4i a0 = lds_read_16(rb + 16 * ((2 * g) ^ sw));
            const v4i a1 = lds_read_16(rb + 16 * ((2 * g + 1) ^ sw));
            const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pk.b, acc, 0, 0, 0, 127, 0, 127);
        } else {
#pragma unroll
            for (int mm = 0; mm < 4; mm++) {
                const v4i araw = lds_read_16(rb + 16 * ((2 * mm + g) ^ sw));
                v8h a;
                __builtin_memcpy(&a, &araw, 16);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pk.b[mm], acc, 0, 0, 0);
            }
        }
        if constexpr (TL) O[dt] += acc;
        else O[dt] = acc;
    }
}

struct KParams {
    const int8_t* q_i8;
    const float* q_scale;
    const int8_t* k_i8;
    const float* k_scale;
    const uint8_t* v_hat;
    const float* v_scale;
    void* out;
    SeqMap qm, km;          // query and key/value sequences (dense or packed batch)
    int64_t osb, osh, osq;  // output element strides (batch, head, token); packed: token = Hq*D, head = D
    int B, Hq, Hkv, G, D, QT;
    int grp;       // causal: kv heads whose query tiles are interleaved (1, 2 or 4)
    float cscale;  // sm_scale * log2(e)
    // key-range splits (SPLIT kernels): split s of a query tile walks key tiles
    // [s * tps, (s + 1) * tps) and leaves its own output O_s / l_s in fp16 in part_o
    // [B*Hq][Nq][splits][Dp] and its running max and row sum in fp32 in part_ml
    // [B*Hq][Nq][splits][2] (Nq = qm.N)
    int splits, tps;
    _Float16* part_o;
    float* part_ml;
    // QF kernels: Q arrives in fp16 / bf16 (q_bf16) with element strides qst, dense batch,
    // and each workgroup quantises its own queries in the prologue; the codes and block
    // scales also go to q_i8_out / q_scale_out where those are non-null
    const uint16_t* q16;
    Strides qst;
    int q_bf16;
    int8_t* q_i8_out;
    float* q_scale_out;
};

// Q quantisation inside the attention prologue (QF): lane (g, i) of a wave loads the
// channels 32 s + 16 g .. + 15 (s < KS) of its query q0 + i -- exactly the bytes of the
// Q operand fragments it holds -- and the two waves of a 64-token block combine their
// maxima through LDS.  The arithmetic is the block quantiser's: amax = max |x| over the
// block's real elements (NaNs ignored), scale = amax / 127, inv = 127 / amax, code =
// clamp(rne(x inv), -127, 127) with a NaN product giving 0; all-zero block: scale 0,
// codes 0.  Absent rows and padding channels load as +0, which changes no maximum and
// gives code 0.
//   The maximum is taken on the magnitude bits: fp16 and bf16 are sign-magnitude, so
// |x| orders like bits & 0x7fff (two values per packed 16-bit maximum); a NaN's bits lie
// above the infinity's, and a block holding one takes the per-element path instead.
//   Codes: with a finite amax and inv, |fp32(x inv)| <= 127 (1 + 2^-23), so the clamp is
// inert and adding 1.5 * 2^23 rounds the product to an integer (ties to even) whose low
// byte is the code (a NaN's low byte is 0: fp16 / bf16 NaNs widen with zero low bits);
// otherwise the clamping path.
template <class C, bool BF16>
__device__ __forceinline__ void quant_q_frags(const KParams& p, v4i (&qf)[C::KS], float& sq, float* blk_amax,
                                              const uint16_t* qbase, int64_t tstride, int q0, int Nq, int64_t row0,
                                              int64_t slot0, int lane, int wave) {
    constexpr int KS = C::KS;
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    const int i = lane & 31, g = lane >> 5;
    const int t = q0 + i;
    const bool row = t < Nq;
    const uint16_t* src = qbase + int64_t(row ? t : 0) * tstride;
    v8u16 raw[KS][2];
    const bool vec = (p.D & 7) == 0;
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int c = 32 * s + 16 * g + 8 * u;
            v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
            if (row && c < p.D) {
                if (vec) {
                    r = *(const v8u16*)(src + c);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++) r[e] = c + e < p.D ? src[c + e] : (unsigned short)0;
                }
            }
            raw[s][u] = r;
        }
    auto word = [&](int s, int w) {  // elements 2w, 2w + 1 of fragment s as one 32-bit word
        const v8u16& r = raw[s][w >> 2];
        return uint32_t(r[2 * (w & 3)]) | (uint32_t(r[2 * (w & 3) + 1]) << 16);
    };
    auto val = [&](int s, int e) { return in_to_f32<BF16>(raw[s][e >> 3][e & 7]); };
    v2u16 mx2 = {0, 0};
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
        for (int w = 0; w < 8; w++) {
            const uint32_t m = word(s, w) & 0x7fff7fffu;
            v2u16 mv;
            __builtin_memcpy(&mv, &m, 4);
            mx2 = __builtin_elementwise_max(mx2, mv);
        }
    const uint32_t mbits = mx2[0] > mx2[1] ? mx2[0] : mx2[1];
    float a;
    if (mbits > (BF16 ? 0x7f80u : 0x7c00u)) {  // a NaN in this lane's elements: fmaxf ignores it
        a = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int e = 0; e < 16; e++) a = fmaxf(a, fabsf(val(s, e)));
    } else {
        a = in_to_f32<BF16>(uint16_t(mbits));
    }
    a = wave_max(a);
    if (lane == 0) blk_amax[wave] = a;
    __syncthreads();
    a = fmaxf(a, blk_amax[wave ^ 1]);
    const bool zero = !(a > 0.0f);
    const float inv = zero ? 0.0f : 127.0f / a;
    sq = zero ? 0.0f : a / 127.0f;
    if (!zero && a <= 3.4e38f && inv <= 3.4e38f) {  // uniform over the two waves of the block
        constexpr float kRound = 12582912.0f;
#pragma unroll
        for (int s = 0; s < KS; s++) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                uint32_t r[4];
#pragma unroll
                for (int e = 0; e < 4; e++) r[e] = __float_as_uint(val(s, 4 * k + e) * inv + kRound);
                w[k] = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u) | __builtin_amdgcn_perm(r[3], r[2], 0x04000c0cu);
            }
            qf[s] = v4i{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
        }
    } else {
#pragma unroll
        for (int s = 0; s < KS; s++) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; e++) {
                int code = 0;
                if (!zero && row && 32 * s + 16 * g + e < p.D) {
                    float r = rintf(val(s, e) * inv);
                    r = r > 127.0f ? 127.0f : r;
                    r = r < -127.0f ? -127.0f : r;
                    code = int(r);
                }
                w[e / 4] |= uint32_t(code & 0xff) << (8 * (e % 4));
            }
            qf[s] = v4i{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
        }
    }
    // the codes and scale for callers that keep them (rows up to the padded block end)
    const int npad = (Nq + kBlk - 1) / kBlk * kBlk;
    if (p.q_i8_out != nullptr && t < npad) {
#pragma unroll
        for (int s = 0; s < KS; s++) *(v4i*)(p.q_i8_out + (row0 + t) * C::KROW + 32 * s + 16 * g) = qf[s];
    }
    if (p.q_scale_out != nullptr && lane == 0 && (wave & 1) == 0 && q0 < npad)
        p.q_scale_out[slot0 + q0 / kBlk] = sq;
}

// TG: the per-thread scales of sage_quant_qkv -- q_scale per token (indexed like the
// rows of q_i8), k_scale per 32 keys ([slot][2]) -- so the dequantisation factor is
// per lane: the lane's query, and its lane half's keys (FP8) or the tile's keys (FP16).
// TL: the explicit two-level P.V accumulation (pv_tile).
// SPLIT: one key range of a query tile (KParams::splits); the fp32 partial state goes to
// the workspace and split_merge_kernel combines the splits.
template <int DP, bool FP8, bool CAUSAL, bool OBF16, bool TG = false, bool TL = false, bool SPLIT = false,
          bool QF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Cfg<DP, FP8>::OCC, Cfg<DP, FP8>::OCC))) void attn_fwd_kernel(KParams p) {
    using C = Cfg<DP, FP8>;
    // NST LDS stages: tile j lives in stage j % NST while tiles j+1 .. j+NST-1 stream in.
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::NST * C::STAGE];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform (SGPR)
    const int g = lane >> 5, i = lane & 31;

    // ---- workgroup -> (b, h, q tile)
    int b, h, qt, sidx = 0;
    block_tile<CAUSAL>(p.B, p.Hkv, p.G, p.QT, p.grp, b, h, qt, SPLIT ? p.splits : 1, &sidx);
    const int hk = h / p.G;
    const SeqView qv = seq_view(p.qm, b, h), kv = seq_view(p.km, b, hk);
    const int Nq = qv.n, Nkv = kv.n, NBk = (Nkv + kBlk - 1) / kBlk;
    if (qt * C::BM >= Nq) return;  // the whole workgroup: past this sequence's queries
    // causal: key j is visible to query i iff j <= i + off (diagonal aligned to the
    // bottom-right corner, so with Nq < Nkv the queries are the sequence's last ones)
    const int off = Nkv - Nq;
    const int q0 = qt * C::BM + wave * C::QW;  // this wave's first query
    const bool active = q0 < Nq;
    const int qb = q0 / kBlk;
    const int qidx = q0 + i;  // this lane's query

    const int8_t* kbase = p.k_i8 + kv.row0 * DP;
    const uint8_t* vbase = p.v_hat + kv.slot0 * C::VBYTES;

    int jend = NBk;
    if constexpr (CAUSAL) {
        const int kmax = min(qt * C::BM + C::BM, Nq) - 1 + off;  // last key the workgroup sees
        jend = kmax < 0 ? 0 : min(NBk, kmax / kBlk + 1);
    }
    // the key tiles this workgroup walks: [jbeg, jend) (all of them unless SPLIT)
    int jbeg = 0;
    if constexpr (SPLIT) {
        jbeg = sidx * p.tps;
        jend = min(jend, jbeg + p.tps);
        jbeg = min(jbeg, jend);  // an empty range leaves m = -1e30, l = 0, O = 0
    }
    const bool ktail = (Nkv % kBlk) != 0;

    // ---- per-wave state
    v4i qf[C::KS];
    float sq = 0.0f;
    if constexpr (QF) {
        // every wave takes part (the block maximum goes through LDS and a barrier)
        __shared__ float blk_amax[C::WAVES];
        // token 0 of this (sequence, head) and the token stride: dense, the input's layout;
        // packed, (total, H_qo, D) as the sequence map describes it
        const bool packed = p.qm.cu != nullptr;
        const uint16_t* qbase = packed ? p.q16 + qv.in_off : p.q16 + b * p.qst.b + h * p.qst.h;
        const int64_t ts = packed ? p.qm.st.t : p.qst.t;
        if (p.q_bf16) quant_q_frags<C, true>(p, qf, sq, blk_amax, qbase, ts, q0, Nq, qv.row0, qv.slot0, lane, wave);
        else quant_q_frags<C, false>(p, qf, sq, blk_amax, qbase, ts, q0, Nq, qv.row0, qv.slot0, lane, wave);
    } else if (active) {
        load_q_frags<C>(qf, p.q_i8 + (qv.row0 + q0) * DP, lane);
        if constexpr (TG) sq = p.q_scale[qv.row0 + qidx];  // 0 for padding rows
        else sq = scalar_load_f32(p.q_scale + qv.slot0 + qb);
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; s++) qf[s] = v4i{0, 0, 0, 0};
    }
    const float* ks_row = p.k_scale + kv.slot0;
    wait_vmcnt<0>();  // Q fragments resident before the tile pipeline starts
    v16f O[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++) O[dt] = v16f{};
    float m = -1e30f, l = 0.0f;

    const DmaPlan<C> dma = make_dma_plan<C>(tid);
    // LDS byte address of this wave's slot in stage 0 (wave-uniform)
    const uint32_t lds_w0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + uint32_t(wave * kWave * 16));
    auto issue_tile = [&](int t) {
        issue_stage<C>(lds_w0 + uint32_t((t % C::NST) * C::STAGE), kbase + int64_t(t) * kBlk * DP,
                       vbase + int64_t(t) * C::VBYTES, dma);
    };
    // tiles [0, jm) need no mask for this wave; [jm, jend) do.  The split is per wave,
    // but every wave runs the same sequence of iterations (and barriers).
    int jm = ktail ? NBk - 1 : NBk;
    if constexpr (CAUSAL) {
        const int seen = q0 + off + 1;  // keys visible to the wave's first query
        jm = min(jm, seen > 0 ? seen / kBlk : 0);
    }
    jm = max(min(jm, jend), jbeg);

    // Tile j lives in stage j % NST; the next NST-1 tiles stream in meanwhile.  Every
    // wave runs every iteration (a fully masked causal tile leaves m, l and O
    // unchanged: p = 0 and all V^ codes, padding included, are finite).
    constexpr int AHEAD = C::NST - 1;  // tiles in flight beyond the current one
    static_assert(AHEAD == 1 || AHEAD == 2, "two or three stages");
#pragma unroll
    for (int t = 0; t < AHEAD; t++)
        if (jbeg + t < jend) issue_tile(jbeg + t);
    // K scale(s) of the next tile, loaded one tile ahead (TG: the two 32-key halves)
    float ks_next = 0.0f, ks_next1 = 0.0f;
    if (jend > jbeg) {
        if constexpr (TG) {
            ks_next = scalar_load_f32(p.k_scale + 2 * (kv.slot0 + jbeg));
            ks_next1 = scalar_load_f32(p.k_scale + 2 * (kv.slot0 + jbeg) + 1);
        } else {
            ks_next = scalar_load_f32(ks_row + jbeg);
        }
    }
    auto step = [&](auto masked, int j) {
        constexpr bool MASK = decltype(masked)::value;
        // tile j landed for this wave (later tiles may still stream); the barrier
        // publishes it for all waves and certifies that iteration j-1, the last
        // reader of the stage refilled below, is over everywhere
        if (AHEAD == 2 && j + 1 < jend) wait_vmcnt<C::ROUNDS>();  // tile j+1 may stream on
        else wait_vmcnt<0>();
        block_barrier();
        if (j + AHEAD < jend) issue_tile(j + AHEAD);
        float c0, c1;
        if constexpr (TG) {
            const float a0 = sq * ks_next * p.cscale, a1 = sq * ks_next1 * p.cscale;
            // FP8: lane half g holds keys 32 g .. 32 g + 31; FP16: tile kt holds 32 kt ..
            c0 = FP8 ? (g ? a1 : a0) : a0;
            c1 = FP8 ? c0 : a1;
            const int jn = min(j + 1, NBk - 1);
            ks_next = scalar_load_f32(p.k_scale + 2 * (kv.slot0 + jn));
            ks_next1 = scalar_load_f32(p.k_scale + 2 * (kv.slot0 + jn) + 1);
        } else {
            c0 = c1 = sq * ks_next * p.cscale;
            ks_next = scalar_load_f32(ks_row + min(j + 1, NBk - 1));
        }
        // a tile no query of this wave may see (causal: beyond the wave's last query's
        // horizon) leaves m, l and O unchanged: take part in the pipeline only
        if constexpr (MASK && CAUSAL)
            if (j * kBlk > q0 + C::QW - 1 + off) return;
        // stage base as one wave-uniform value, so each LDS address costs a single add
        const uint8_t* st = smem + __builtin_amdgcn_readfirstlane((j % C::NST) * C::STAGE);
        v16i S[2];
        qk_tile<C, FP8, (DP <= 128)>(st, qf, S, lane);
        PPack<FP8> pk;
        const float alpha =
            softmax_tile<FP8, MASK, CAUSAL, TG && !FP8, (DP <= 128)>(S, pk, c0, c1, m, l, g, j * kBlk, qidx + off, Nkv);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < C::DT; dt++) O[dt] *= alpha;
        }
        pv_tile<C, FP8, TL>(st + C::KBYTES, pk, O, lane);
    };
    int j = jbeg;
    for (; j < jm; j++) step(std::false_type{}, j);
    for (; j < jend; j++) step(std::true_type{}, j);
    // Matrix instructions must run with every lane enabled: without these empty uses the
    // compiler sinks the last P.V MFMAs into the epilogue, below the per-lane exit of
    // padding queries, and the operand rows held by the exited lanes are lost.
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++) asm volatile("" : "+v"(O[dt]));

    // ---- epilogue: O^T / l (x v_scale in FP8 mode) -> out dtype, input layout
    if (!active) return;
    const float ltot = halves_sum(l);
    if constexpr (SPLIT) {
        // this split's own output O / l in fp16 (all Dp channels; padding ones are 0; zeros
        // for an empty range), its running max and row sum in fp32.  |O / l| is bounded by
        // the largest |v^|, an fp16 value, so the fp16 store cannot overflow.
        if (qidx >= Nq) return;
        const int64_t row = ((int64_t(b) * p.Hq + h) * p.qm.N + qidx) * p.splits + sidx;
        const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
        _Float16* po = p.part_o + row * DP;
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
            for (int a4 = 0; a4 < 4; a4++) {
                const int k0 = 4 * a4;
                *(uint2*)(po + 32 * dt + 8 * a4 + 4 * g) =
                    make_uint2(uint32_t(f32_to_f16_bits(O[dt][k0] * inv)) |
                                   (uint32_t(f32_to_f16_bits(O[dt][k0 + 1] * inv)) << 16),
                               uint32_t(f32_to_f16_bits(O[dt][k0 + 2] * inv)) |
                                   (uint32_t(f32_to_f16_bits(O[dt][k0 + 3] * inv)) << 16));
            }
        if (g == 0) *(v2f*)(p.part_ml + row * 2) = v2f{m, ltot};
        return;
    }
    const bool empty = !(ltot > 0.0f);  // a query that sees no key: zeros
    const float inv = empty ? 0.0f : 1.0f / ltot;
    if (qidx >= Nq) return;
    // FP8: the V scales ([B][H_kv][Dp], so every padded channel is in bounds) of a group of
    // the lane's channels -- all 64 at head dims up to 128 -- loaded before the group's
    // first store: interleaved with the stores (which might alias them) each load would
    // wait out its own latency, 64 times per workgroup
    constexpr int DTG = DP <= 128 ? C::DT : 2;  // 32-channel tiles per group
    const float* vsc = FP8 ? p.v_scale + (int64_t(b) * p.Hkv + hk) * DP : nullptr;
    const bool vec4 = (p.D & 3) == 0;
    const int64_t obase = p.qm.cu != nullptr ? qv.start * p.osq : b * p.osb;
    uint16_t* orow = (uint16_t*)p.out + obase + h * p.osh + qidx * p.osq;
#pragma unroll
    for (int dg = 0; dg < C::DT; dg += DTG) {
        float vs[FP8 ? DTG : 1][4][4];
        if constexpr (FP8) {
#pragma unroll
            for (int u = 0; u < DTG; u++)
#pragma unroll
                for (int a4 = 0; a4 < 4; a4++)
#pragma unroll
                    for (int e = 0; e < 4; e++) vs[u][a4][e] = vsc[32 * (dg + u) + 8 * a4 + 4 * g + e];
        }
#pragma unroll
        for (int u = 0; u < DTG; u++)
#pragma unroll
            for (int a4 = 0; a4 < 4; a4++) {
                const int dt = dg + u, d0 = 32 * dt + 8 * a4 + 4 * g;
                if (d0 >= p.D) continue;
                uint16_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    float o = O[dt][4 * a4 + e] * inv;
                    if constexpr (FP8) o = empty ? 0.0f : o * vs[u][a4][e];
                    hv[e] = OBF16 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o);
                }
                if (vec4) {
                    *(uint2*)(orow + d0) = make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16),
                                                      uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        if (d0 + e < p.D) orow[d0 + e] = hv[e];
                }
            }
    }
}

// ---- combining key-range splits ----------------------------------------------------
// One thread per (b, h, query, 8 channels): the splits' states (o_s = O_s / l_s, m_s, l_s)
// combine as o = sum_s w_s o_s / sum_s w_s with w_s = 2^(m_s - M) l_s and M = max_s m_s
// (fp32), times v_scale / 448 in FP8 mode, then the output dtype and layout of the
// unsplit kernel.  The splits are taken four at a time, all loads of a group issued
// before any use; a later group with a larger maximum rescales what the earlier ones
// summed (with at most four splits, one group: M is the maximum over all of them).  A
// query with no visible key (every l_s = 0) gets zeros.
template <int DP, bool FP8, bool OBF16>
__global__ __launch_bounds__(256) void split_merge_kernel(KParams p) {
    constexpr int G8 = DP / 8;
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t r = t / G8;
    const int d0 = int(t % G8) * 8;
    const int NqM = p.qm.N;
    if (r >= int64_t(p.B) * p.Hq * NqM || d0 >= p.D) return;
    const int q = int(r % NqM), bh = int(r / NqM), b = bh / p.Hq, h = bh % p.Hq;
    const SeqView qv = seq_view(p.qm, b, h);
    if (q >= qv.n) return;
    const float* ml = p.part_ml + r * p.splits * 2;
    const _Float16* po = p.part_o + r * p.splits * DP + d0;
    float M = -1e30f, L = 0.0f;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < p.splits; s0 += 4) {
        v2f st[4];
        uint4 ov[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const bool in = s0 + u < p.splits;
            st[u] = in ? *(const v2f*)(ml + 2 * (s0 + u)) : v2f{-1e30f, 0.0f};
            ov[u] = in ? *(const uint4*)(po + (s0 + u) * DP) : make_uint4(0, 0, 0, 0);
        }
        const float Mn = fmaxf(fmaxf(fmaxf(M, st[0].x), fmaxf(st[1].x, st[2].x)), st[3].x);
        const float sc = __builtin_amdgcn_exp2f(M - Mn);  // 0 on the first group
        L *= sc;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[e] *= sc;
        M = Mn;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const float w = __builtin_amdgcn_exp2f(st[u].x - M) * st[u].y;  // 0 for an empty or absent split
            L += w;
            const uint32_t wd[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w};
#pragma unroll
            for (int e = 0; e < 8; e++)
                acc[e] = __builtin_fmaf(w, f16_bits_to_f32(uint16_t(wd[e >> 1] >> (16 * (e & 1)))), acc[e]);
        }
    }
    const bool empty = !(L > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / L;
    const int hk = h / p.G;
    const int64_t obase = p.qm.cu != nullptr ? qv.start * p.osq : b * p.osb;
    uint16_t* orow = (uint16_t*)p.out + obase + h * p.osh + q * p.osq;
    uint16_t hv[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        float o = acc[e] * inv;
        if constexpr (FP8) o = empty ? 0.0f : o * p.v_scale[(int64_t(b) * p.Hkv + hk) * DP + d0 + e];
        hv[e] = OBF16 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o);
    }
    auto pack = [&](int e) { return uint32_t(hv[e]) | (uint32_t(hv[e + 1]) << 16); };
    if ((p.D & 7) == 0) {
        *(uint4*)(orow + d0) = make_uint4(pack(0), pack(2), pack(4), pack(6));
    } else if ((p.D & 3) == 0) {
        *(uint2*)(orow + d0) = make_uint2(pack(0), pack(2));
        if (d0 + 4 < p.D) *(uint2*)(orow + d0 + 4) = make_uint2(pack(4), pack(6));
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            if (d0 + e < p.D) orow[d0 + e] = hv[e];
    }
}

// ---- debug dump of INT32 score tiles through the same loader / operand path ----------
// One workgroup per tile: the K^ tile arrives through the attention kernel's own
// direct-to-LDS plan (its K^ rounds: same per-thread offsets, swizzle, waits and
// barrier); waves 0 and 1 compute the two 32-query halves with qk_tile in the
// accumulator form the attention kernel uses (offset scores at head dims up to 128,
// whose bias is taken off as an integer before the write).
template <int DP, bool FP8>
__global__ __launch_bounds__(256) void debug_qk_kernel(const int8_t* __restrict__ q_i8,
                                                       const int8_t* __restrict__ k_i8, int B, int Hq, int Hkv,
                                                       int NBq, int NBk, const int32_t* __restrict__ tiles,
                                                       int32_t* __restrict__ out) {
    using C = Cfg<DP, FP8>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::STAGE];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int b = tiles[4 * t], h = tiles[4 * t + 1], qb = tiles[4 * t + 2], kb = tiles[4 * t + 3];
    int32_t* o = out + int64_t(t) * kBlk * kBlk;
    const bool ok = b >= 0 && b < B && h >= 0 && h < Hq && qb >= 0 && qb < NBq && kb >= 0 && kb < NBk;
    if (!ok) {  // out-of-range tuple: fill with INT32_MIN, touch nothing else
        for (int e = tid; e < kBlk * kBlk; e += C::THREADS) o[e] = INT32_MIN;
        return;
    }
    constexpr bool OFS = DP <= 128;
    const int hk = h / (Hq / Hkv);
    const int8_t* ktile = k_i8 + ((int64_t(b) * Hkv + hk) * NBk + kb) * kBlk * DP;
    const DmaPlan<C> dma = make_dma_plan<C>(tid);
    const uint32_t lds_w0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + uint32_t(wave * kWave * 16));
    issue_stage<C, 0, C::KROUNDS>(lds_w0, ktile, nullptr, dma);
    wait_vmcnt<0>();
    block_barrier();
    if (wave >= 2) return;
    v4i qf[C::KS];
    load_q_frags<C>(qf, q_i8 + (((int64_t(b) * Hq + h) * NBq + qb) * kBlk + wave * C::QW) * DP, lane);
    v16i S[2];
    qk_tile<C, FP8, OFS>(smem, qf, S, lane);
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            o[(wave * C::QW + i) * kBlk + key_of_reg<FP8>(kt, g, r)] = OFS ? S[kt][r] - kScoreBias : S[kt][r];
}

template <int DP, bool FP8, bool CAUSAL, bool OBF16, bool TG, bool TL = false, bool QF = false>
hipError_t launch_attn_t(const KParams& p, int nwg, hipStream_t s) {
    using C = Cfg<DP, FP8>;
    auto kern = attn_fwd_kernel<DP, FP8, CAUSAL, OBF16, TG, TL, false, QF>;
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(C::THREADS), 0, s, p);
    return hipGetLastError();
}

// key-range splits (FP16 P.V, block granularity): the split kernel, then the merge
template <int DP>
hipError_t dispatch_split(const AttnArgs& a, const KParams& p, int nwg, hipStream_t s) {
    using C = Cfg<DP, false>;
    if (a.causal)
        hipLaunchKernelGGL((attn_fwd_kernel<DP, false, true, false, false, false, true>), dim3(nwg), dim3(C::THREADS),
                           0, s, p);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<DP, false, false, false, false, false, true>), dim3(nwg),
                           dim3(C::THREADS), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = int64_t(p.B) * p.Hq * p.qm.N * (DP / 8);
    const dim3 grid(unsigned((threads + 255) / 256));
    if (a.out_bf16)
        hipLaunchKernelGGL((split_merge_kernel<DP, false, true>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((split_merge_kernel<DP, false, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// Q quantised in the attention prologue (block granularity, dense batches)
template <int DP, bool FP8>
hipError_t dispatch_qf(const AttnArgs& a, const KParams& p, int nwg, hipStream_t s) {
    const int key = (a.causal ? 2 : 0) | (a.out_bf16 ? 1 : 0);
    switch (key) {
    case 0: return launch_attn_t<DP, FP8, false, false, false, false, true>(p, nwg, s);
    case 1: return launch_attn_t<DP, FP8, false, true, false, false, true>(p, nwg, s);
    case 2: return launch_attn_t<DP, FP8, true, false, false, false, true>(p, nwg, s);
    default: return launch_attn_t<DP, FP8, true, true, false, false, true>(p, nwg, s);
    }
}

template <int DP, bool FP8>
hipError_t dispatch_rest(const AttnArgs& a, const KParams& p, int nwg, hipStream_t s) {
    // SAGE_ACC_FP32 and SAGE_ACC_FP16_FP32 both run the accumulation straight into O
    // (fp32 at every level already); the literal two-level form runs for
    // SAGE_ACC_FP16_FP32_SPLIT
    if (a.split_partials) {
        const int k2 = (a.causal ? 2 : 0) | (a.out_bf16 ? 1 : 0);
        switch (k2) {
        case 0: return launch_attn_t<DP, FP8, false, false, false, true>(p, nwg, s);
        case 1: return launch_attn_t<DP, FP8, false, true, false, true>(p, nwg, s);
        case 2: return launch_attn_t<DP, FP8, true, false, false, true>(p, nwg, s);
        default: return launch_attn_t<DP, FP8, true, true, false, true>(p, nwg, s);
        }
    }
    const int key = (a.thread_gran ? 4 : 0) | (a.causal ? 2 : 0) | (a.out_bf16 ? 1 : 0);
    switch (key) {
    case 0: return launch_attn_t<DP, FP8, false, false, false>(p, nwg, s);
    case 1: return launch_attn_t<DP, FP8, false, true, false>(p, nwg, s);
    case 2: return launch_attn_t<DP, FP8, true, false, false>(p, nwg, s);
    case 3: return launch_attn_t<DP, FP8, true, true, false>(p, nwg, s);
    case 4: return launch_attn_t<DP, FP8, false, false, true>(p, nwg, s);
    case 5: return launch_attn_t<DP, FP8, false, true, true>(p, nwg, s);
    case 6: return launch_attn_t<DP, FP8, true, false, true>(p, nwg, s);
    default: return launch_attn_t<DP, FP8, true, true, true>(p, nwg, s);
    }
}

template <int DP, bool FP8>
hipError_t launch_debug_t(const DebugQKArgs& a, int NBq, int NBk, hipStream_t s) {
    using C = Cfg<DP, FP8>;
    auto kern = debug_qk_kernel<DP, FP8>;
    hipLaunchKernelGGL(kern, dim3(a.T), dim3(C::THREADS), 0, s, a.q_i8, a.k_i8, a.B, a.Hq, a.Hkv, NBq, NBk, a.tiles,
                       a.out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s) {
    KParams p;
    p.q_i8 = a.q_i8;
    p.q_scale = a.q_scale;
    p.k_i8 = a.k_i8;
    p.k_scale = a.k_scale;
    p.v_hat = (const uint8_t*)a.v_hat;
    p.v_scale = a.v_scale;
    p.out = a.out;
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.D = a.D;
    // the quantised operands' rows and slots (their input layout plays no part here)
    p.qm = make_seq_map(0, a.cu_q, a.B, a.Hq, a.Nq, a.total_q, a.D);
    p.km = make_seq_map(0, a.cu_k, a.B, a.Hkv, a.Nkv, a.total_k, a.D);
    constexpr int BM = Cfg<128, true>::BM;
    static_assert(Cfg<64, false>::BM == BM && Cfg<64, true>::BM == BM && Cfg<128, false>::BM == BM &&
                      Cfg<256, true>::BM == BM && Cfg<256, false>::BM == BM,
                  "uniform BM");
    p.QT = (a.Nq + BM - 1) / BM;
    const int dp = a.D <= 64 ? 64 : (a.D <= 128 ? 128 : 256);
    const int64_t head_bytes = int64_t((a.Nkv + kBlk - 1) / kBlk) * kBlk * dp * (a.fp8 ? 2 : 3);  // K^ + V^
    p.grp = causal_head_group(head_bytes, int64_t(a.B) * a.Hq * p.QT, int64_t(p.G) * p.QT);
    p.cscale = a.sm_scale * kLog2e;
    if (a.cu_q != nullptr) {  // packed (total, H_qo, D)
        p.osb = 0;
        p.osh = a.D;
        p.osq = int64_t(a.Hq) * a.D;
    } else if (a.out_nhd) {
        p.osb = int64_t(a.Nq) * a.Hq * a.D;
        p.osh = a.D;
        p.osq = int64_t(a.Hq) * a.D;
    } else {
        p.osb = int64_t(a.Hq) * a.Nq * a.D;
        p.osh = int64_t(a.Nq) * a.D;
        p.osq = a.D;
    }
    const int nwg = a.B * a.Hq * p.QT;
    p.splits = 1;
    p.tps = 0;
    p.part_o = nullptr;
    p.part_ml = nullptr;
    p.q16 = (const uint16_t*)a.q16;
    p.qst = make_strides(a.q_nhd, a.Hq, a.Nq, a.D);
    p.q_bf16 = a.q_bf16;
    p.q_i8_out = a.q_i8_out;
    p.q_scale_out = a.q_scale_out;
    if (a.q16 != nullptr) {
        if (a.D <= 64) return a.fp8 ? dispatch_qf<64, true>(a, p, nwg, s) : dispatch_qf<64, false>(a, p, nwg, s);
        if (a.D <= 128) return a.fp8 ? dispatch_qf<128, true>(a, p, nwg, s) : dispatch_qf<128, false>(a, p, nwg, s);
        return a.fp8 ? dispatch_qf<256, true>(a, p, nwg, s) : dispatch_qf<256, false>(a, p, nwg, s);
    }
    if (a.splits > 1) {
        // balanced ranges: tps key tiles each, as few splits as cover every key tile
        const int NBk = (a.Nkv + kBlk - 1) / kBlk;
        p.tps = (NBk + a.splits - 1) / a.splits;
        p.splits = (NBk + p.tps - 1) / p.tps;
        const SplitWorkspace ws = attn_split_workspace(a.B, a.Hq, a.Nq, a.D, a.splits);
        p.part_o = (_Float16*)a.workspace;
        p.part_ml = (float*)((char*)a.workspace + ws.ml);
        if (p.splits > 1) {
            const int n = nwg * p.splits;
            p.grp = causal_head_group(head_bytes, n, int64_t(p.G) * p.QT * p.splits);
            if (a.D <= 64) return dispatch_split<64>(a, p, n, s);
            if (a.D <= 128) return dispatch_split<128>(a, p, n, s);
            return dispatch_split<256>(a, p, n, s);
        }
        p.splits = 1;
    }
    if (a.D <= 64) return a.fp8 ? dispatch_rest<64, true>(a, p, nwg, s) : dispatch_rest<64, false>(a, p, nwg, s);
    if (a.D <= 128) return a.fp8 ? dispatch_rest<128, true>(a, p, nwg, s) : dispatch_rest<128, false>(a, p, nwg, s);
    return a.fp8 ? dispatch_rest<256, true>(a, p, nwg, s) : dispatch_rest<256, false>(a, p, nwg, s);
}

hipError_t launch_debug_qk(const DebugQKArgs& a, hipStream_t s) {
    const int NBq = (a.Nq + kBlk - 1) / kBlk, NBk = (a.Nkv + kBlk - 1) / kBlk;
    if (a.D <= 64) return a.fp8 ? launch_debug_t<64, true>(a, NBq, NBk, s) : launch_debug_t<64, false>(a, NBq, NBk, s);
    if (a.D <= 128) return a.fp8 ? launch_debug_t<128, true>(a, NBq, NBk, s) : launch_debug_t<128, false>(a, NBq, NBk, s);
    return a.fp8 ? launch_debug_t<256, true>(a, NBq, NBk, s) : launch_debug_t<256, false>(a, NBq, NBk, s);
}

}  // namespace sage
