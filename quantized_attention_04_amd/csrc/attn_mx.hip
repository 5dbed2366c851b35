// attn_mx.hip -- microscaling FP4 attention forward for gfx950.
//
// Method: the SageAttention project README names a microscaling FP4 attention
// ("SageAttention3: Microscaling FP4 Attention for Inference", project updates and
// citations) and gives only that title.  This kernel takes the OCP MX v1.0 MXFP4
// format that gfx950's scaled matrix instructions read, applied to both products of
// the INT8 scheme (see include/sage.h, "Microscaling FP4"):
//   S   = sum over channels of Q^ K^ with one power-of-two scale per 32 channels of
//         each query and of each (smoothed) key, on v_mfma_scale_f32_32x32x64_f8f6f4
//         in FP4 mode -- the scales are applied inside the matrix instruction, so the
//         scores arrive in fp32;
//   t   = fma(S, c, -m), c = sm_scale * log2(e), m the running max of S c over 64-key
//         tiles rounded toward -inf, so that the row maximum has 0 <= t < one ulp of m
//         and p = 1 (to 2^-20, never below 1: a p of the maximum just below 1 would
//         give its P block the next lower exponent and clip it from 8 X to 6 X);
//         p = 2^t; l = alpha * l + sum p (unquantised);
//   P^  = e2m1(p / X) per 32 keys (one lane's keys), X = 2^(floor(log2 pmax) - 2);
//   O   = alpha * O + P^ V^ on the same instruction with P's and V's scales.
//
// gfx950 design (shared with the INT8 kernel): workgroup = 4 waves = 128 queries; a
// wave owns 32 queries and walks 64-key tiles; K^/V^ tiles (half the bytes of INT8 /
// FP8) and their exponent bytes stream HBM -> LDS with direct-to-LDS loads two tiles
// ahead; S^T = K^ Q^T with keys on the M side, rows permuted so that the score
// registers are the P.V B operand: lane half g holds keys 32 g .. 32 g + 31 -- exactly
// one MX block of P per lane, so P's block maximum and scale are lane-local.
#include "common.hpp"
#include "internal.hpp"

#include <utility>

namespace sage {

namespace {

template <int DP>
struct MXCfg {
    static constexpr int WAVES = 4;
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int QW = 32;               // queries per wave
    static constexpr int BM = WAVES * QW;       // queries per workgroup
    static constexpr int NE = DP / 32;          // exponent bytes per row (one per 32 channels)
    static constexpr int KROW = DP / 2;         // K^ code bytes per key
    static constexpr int VROW = kBlk / 2;       // V^ code bytes per channel (64 keys)
    static constexpr int KBYTES = kBlk * KROW;
    static constexpr int VBYTES = DP * VROW;
    static constexpr int KEXP = kBlk * NE;      // K exponents of a tile [key][NE]
    static constexpr int VEXP = 2 * DP;         // V exponents of a tile [half][channel % 32][channel / 32]
    static constexpr int EXB = KEXP + VEXP;     // = 4 DP: each wave copies DP bytes of it
    static constexpr int ELANES = DP / 16;      // lanes of a wave that copy exponents
    static constexpr int ROUNDS = (KBYTES + VBYTES) / (THREADS * 16);  // code rounds per thread
    static constexpr int LOADS = ROUNDS + 1;    // direct-to-LDS loads per thread per tile
    static constexpr int STAGE = KBYTES + VBYTES + EXB;
    static constexpr int KS = DP / 64;          // QK^T instructions per score tile
    static constexpr int DT = DP / 32;          // 32-channel tiles of O^T
    static constexpr int OCC = DP == 64 ? 4 : (DP == 128 ? 3 : 2);  // head dim 256: 128 accumulator VGPRs
    static constexpr int NST = 3;
    static_assert((KBYTES + VBYTES) % (THREADS * 16) == 0 && KBYTES % (kWave * 16) == 0,
                  "every wave's 1 KB of a code round lies in one region");
    static_assert(KEXP % (ELANES * 16) == 0, "every wave's exponent bytes lie in one region");
};

// XOR swizzles of the 16-byte chunks of a row, chosen so that the operand reads (8 lanes
// x 128 B or 16 lanes x 256 B served per LDS cycle) hit distinct banks:
//  K^ (head dim 256: 8 chunks per key; 128: 4; 64: 2), read at keys key_of_row(kt, i)
//  -- the 8 (16) lanes of a cycle read keys that differ in bits 0, 1, 5 (1, 2, 5);
//  V^ (2 chunks per channel), read at channels 32 t + i.
template <int DP>
__device__ __forceinline__ int mx_kswz(int row) {
    if constexpr (DP == 256) return ((row ^ (row >> 2)) & 1) | (row & 2) | (((row >> 5) & 1) << 2);
    else if constexpr (DP == 128) return (((row >> 1) ^ (row >> 2)) & 1) | (((row >> 5) & 1) << 1);
    else return (row >> 5) & 1;
}
__device__ __forceinline__ int mx_vswz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// Key (0..63) whose K^ row feeds row i of score tile kt: lane half g, register r of
// the result then holds key 32 g + 16 kt + r, the order of the P.V B operand.
__device__ __forceinline__ int mx_key_of_row(int kt, int i) {
    const int a = i >> 3, g = (i >> 2) & 1, b = i & 3;
    return 32 * g + 16 * kt + 4 * a + b;
}

template <int DP>
struct MXDma {
    uint32_t off[MXCfg<DP>::ROUNDS];  // byte offsets of this thread's code chunks in the tile's K^ or V^
    uint32_t eoff;                    // byte offset of its exponent chunk (lanes < ELANES)
};
template <int DP>
__device__ __forceinline__ MXDma<DP> mx_dma_plan(int tid) {
    using C = MXCfg<DP>;
    MXDma<DP> d;
#pragma unroll
    for (int u = 0; u < C::ROUNDS; u++) {
        const int ci = u * C::THREADS + tid;
        if (ci * 16 < C::KBYTES) {
            const int row = ci / (C::KROW / 16), pos = ci % (C::KROW / 16);
            d.off[u] = uint32_t(row * C::KROW + 16 * (pos ^ mx_kswz<DP>(row)));
        } else {
            const int vi = ci - C::KBYTES / 16;
            const int row = vi / 2, pos = vi % 2;
            d.off[u] = uint32_t(row * C::VROW + 16 * (pos ^ mx_vswz(row)));
        }
    }
    // exponents: wave w copies bytes [w DP, (w + 1) DP) of the K-then-V exponent record
    const int w = tid / kWave, l = tid % kWave;
    const int e = w * DP + 16 * l;
    d.eoff = uint32_t(e < C::KEXP ? e : e - C::KEXP);
    return d;
}

struct MXParams {
    const uint8_t* q4;
    const uint8_t* q4_exp;
    const uint8_t* k4;
    const uint8_t* k4_exp;
    const uint8_t* v4;
    const uint8_t* v4_exp;
    void* out;
    SeqMap qm, km;
    int64_t osb, osh, osq;
    int B, Hq, Hkv, G, D, QT;
    int grp;       // causal: kv heads whose query tiles are interleaved (1, 2 or 4)
    float cscale;  // sm_scale * log2(e)
    // QF kernels: Q in fp16 / bf16 (q_bf16) with element strides qst, dense batch,
    // quantised by each lane in the prologue; the codes and exponent bytes also go to
    // q4_out / q4_exp_out where those are non-null
    const uint16_t* q16;
    Strides qst;
    int q_bf16;
    uint8_t* q4_out;
    uint8_t* q4_exp_out;
};

// three-input maximum of scores straight from the matrix instruction: the
// NaN-propagating maximum needs no quieting of its inputs (fmaxf would add one
// instruction per pair)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// f(integral_constant<0>) .. f(integral_constant<N - 1>): the byte selects of the scaled
// matrix instruction are immediates, so loops that pick one exponent byte per step are
// unrolled at compile time
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// NE exponent bytes (2, 4 or 8) from LDS as 32-bit words, byte n in byte n % 4 of word n / 4
template <int NE>
__device__ __forceinline__ void load_exp_words(const uint8_t* p, uint32_t (&w)[(NE + 3) / 4]) {
    if constexpr (NE == 2) {
        w[0] = *(const uint16_t*)p;
    } else if constexpr (NE == 4) {
        w[0] = *(const uint32_t*)p;
    } else {
        const uint2 x = *(const uint2*)p;
        w[0] = x.x;
        w[1] = x.y;
    }
}

__device__ __forceinline__ int mx_exp_dev(float amax) {  // floor(log2 amax) - 2, at least -126
    return max(int((__float_as_uint(amax) >> 23) & 0xffu) - 129, -126);
}

// MXFP4 Q inside the attention prologue (QF): every block of 32 channels of a query is
// exactly the 32 k-values one lane holds for one matrix-instruction k-step (channels
// 64 s + 32 g .. + 31 of query qidx), so each lane quantises its own blocks with no
// exchange, in the arithmetic of the separate quantiser: amax = max |x| over the block's
// real elements (absent rows and padding channels are +0), E = floor(log2 amax) - 2
// held to [-126, 127], codes e2m1(x / 2^E) by the scaled conversion (round to nearest
// even, saturating at 6), element 2t in the low nibble of byte t.
template <class C, bool BF16>
__device__ __forceinline__ void mx_quant_q(const MXParams& p, v4i (&qf)[C::KS], int (&qsc)[C::KS], int b, int h,
                                           int qidx, int Nq, int64_t row0, int g) {
    const bool row = qidx < Nq;
    const uint16_t* src = p.q16 + b * p.qst.b + h * p.qst.h + int64_t(row ? qidx : 0) * p.qst.t;
    const bool vec = (p.D & 7) == 0;
#pragma unroll
    for (int s = 0; s < C::KS; s++) {
        float y[32];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int c = 64 * s + 32 * g + 8 * u;
            v8u16 r = {0, 0, 0, 0, 0, 0, 0, 0};
            if (row && c < p.D) {
                if (vec) {
                    r = *(const v8u16*)(src + c);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++) r[e] = c + e < p.D ? src[c + e] : (unsigned short)0;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; e++) y[8 * u + e] = in_to_f32<BF16>(r[e]);
        }
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; e++) am = fmaxf(am, fabsf(y[e]));
        const int E = mx_exp_dev(am);
        const float X = __uint_as_float(uint32_t(E + 127) << 23);
        int wd[4];
#pragma unroll
        for (int w = 0; w < 4; w++) {
            int x = 0;
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * w + 0], y[8 * w + 1], X, 0);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * w + 2], y[8 * w + 3], X, 1);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * w + 4], y[8 * w + 5], X, 2);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, y[8 * w + 6], y[8 * w + 7], X, 3);
            wd[w] = x;
        }
        qf[s] = v4i{wd[0], wd[1], wd[2], wd[3]};
        qsc[s] = E + 127;
    }
    // the codes and exponent bytes for callers that keep them (rows up to the padded
    // block end; a padding row quantises +0: codes 0, exponent byte 1)
    const int npad = (Nq + kBlk - 1) / kBlk * kBlk;
    if (qidx < npad) {
        if (p.q4_out != nullptr) {
#pragma unroll
            for (int s = 0; s < C::KS; s++) *(v4i*)(p.q4_out + (row0 + qidx) * C::KROW + 32 * s + 16 * g) = qf[s];
        }
        if (p.q4_exp_out != nullptr) {
#pragma unroll
            for (int s = 0; s < C::KS; s++) p.q4_exp_out[(row0 + qidx) * C::NE + 2 * s + g] = uint8_t(qsc[s]);
        }
    }
}

template <int DP, bool CAUSAL, bool OBF16, bool QF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MXCfg<DP>::OCC, MXCfg<DP>::OCC))) void
attn_mx_kernel(MXParams p) {
    using C = MXCfg<DP>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::NST * C::STAGE];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 5, i = lane & 31;

    int b, h, qt;
    block_tile<CAUSAL>(p.B, p.Hkv, p.G, p.QT, p.grp, b, h, qt);
    const int hk = h / p.G;
    const SeqView qv = seq_view(p.qm, b, h), kv = seq_view(p.km, b, hk);
    const int Nq = qv.n, Nkv = kv.n, NBk = (Nkv + kBlk - 1) / kBlk;
    if (qt * C::BM >= Nq) return;
    const int off = Nkv - Nq;  // causal: key j visible to query i iff j <= i + off
    const int q0 = qt * C::BM + wave * C::QW;
    const bool active = q0 < Nq;
    const int qidx = q0 + i;

    const uint8_t* kbase = p.k4 + kv.row0 * C::KROW;
    const uint8_t* vbase = p.v4 + kv.slot0 * C::VBYTES;
    const uint8_t* kebase = p.k4_exp + kv.row0 * C::NE;
    const uint8_t* vebase = p.v4_exp + kv.slot0 * C::VEXP;

    int jend = NBk;
    if constexpr (CAUSAL) {
        const int kmax = min(qt * C::BM + C::BM, Nq) - 1 + off;
        jend = kmax < 0 ? 0 : min(NBk, kmax / kBlk + 1);
    }
    const bool ktail = (Nkv % kBlk) != 0;

    // Q codes (16 bytes per 64-channel step) and the scale byte of each step for this
    // lane: block 2 s + g of the lane's query
    v4i qf[C::KS];
    int qsc[C::KS];
    if constexpr (QF) {
        if (p.q_bf16) mx_quant_q<C, true>(p, qf, qsc, b, h, qidx, Nq, qv.row0, g);
        else mx_quant_q<C, false>(p, qf, qsc, b, h, qidx, Nq, qv.row0, g);
    } else if (active) {
        const uint8_t* qrow = p.q4 + (qv.row0 + qidx) * C::KROW;
        const uint8_t* qe = p.q4_exp + (qv.row0 + qidx) * C::NE;
#pragma unroll
        for (int s = 0; s < C::KS; s++) {
            qf[s] = *(const v4i*)(qrow + 32 * s + 16 * g);
            qsc[s] = qe[2 * s + g];
        }
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; s++) {
            qf[s] = v4i{0, 0, 0, 0};
            qsc[s] = 127;
        }
    }
    wait_vmcnt<0>();
    v16f O[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++) O[dt] = v16f{};
    float m = -1e30f, l = 0.0f;
    const float c = p.cscale;

    const MXDma<DP> dma = mx_dma_plan<DP>(tid);
    const uint32_t lds_w0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + uint32_t(wave * kWave * 16));
    const bool kexp_wave = wave * DP < C::KEXP;  // wave-uniform: this wave copies K (else V) exponents
    auto issue_tile = [&](int t) {
        const uint32_t st = lds_w0 + uint32_t((t % C::NST) * C::STAGE);
#pragma unroll
        for (int u = 0; u < C::ROUNDS; u++) {
            const bool kreg = (u * C::THREADS + wave * kWave) * 16 < C::KBYTES;  // wave-uniform
            const void* base = kreg ? (const void*)(kbase + int64_t(t) * C::KBYTES)
                                    : (const void*)(vbase + int64_t(t) * C::VBYTES);
            // chunk u * THREADS + tid lands at byte 16 (u * THREADS + tid) of the stage
            const uint32_t dst = st + uint32_t(u * C::THREADS * 16);
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(dma.off[u]), "s"(base), "{m0}"(dst) : "memory");
        }
        // the exponent record sits after the codes: wave w's DP bytes at KBYTES + VBYTES + w DP
        const void* ebase = kexp_wave ? (const void*)(kebase + int64_t(t) * C::KEXP)
                                      : (const void*)(vebase + int64_t(t) * C::VEXP);
        const uint32_t edst = lds_addr(smem) + uint32_t((t % C::NST) * C::STAGE + C::KBYTES + C::VBYTES + wave * DP);
        if (lane < C::ELANES)
            asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(dma.eoff), "s"(ebase),
                         "{m0}"(__builtin_amdgcn_readfirstlane(edst))
                         : "memory");
    };
    int jm = ktail ? NBk - 1 : NBk;
    if constexpr (CAUSAL) {
        const int seen = q0 + off + 1;
        jm = min(jm, seen > 0 ? seen / kBlk : 0);
    }
    jm = min(jm, jend);

    if (jend > 0) issue_tile(0);
    if (jend > 1) issue_tile(1);

    auto step = [&](auto masked, int j) {
        constexpr bool MASK = decltype(masked)::value;
        if (j + 1 < jend) wait_vmcnt<C::LOADS>();  // tile j landed; tile j + 1 may stream on
        else wait_vmcnt<0>();
        block_barrier();
        if (j + 2 < jend) issue_tile(j + 2);
        if constexpr (MASK && CAUSAL)
            if (j * kBlk > q0 + C::QW - 1 + off) return;
        const uint8_t* st = smem + __builtin_amdgcn_readfirstlane((j % C::NST) * C::STAGE);
        const uint8_t* kex = st + C::KBYTES + C::VBYTES;
        const uint8_t* vex = kex + C::KEXP;

        // ---- S^T = K^ Q^T (fp32, block scales applied by the instruction)
        v16f S[2];
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            const int row = mx_key_of_row(kt, i);
            const int sw = mx_kswz<DP>(row);
            const uint8_t* rbase = st + row * C::KROW;
            // the row's exponent bytes 2 s + g (this lane half's blocks) moved to bytes 2 s:
            // k-step s takes byte 2 (s % 2) of word s / 2 through the instruction's byte select
            uint32_t kw[(C::NE + 3) / 4];
            load_exp_words<C::NE>(kex + row * C::NE, kw);
#pragma unroll
            for (int u = 0; u < (C::NE + 3) / 4; u++) kw[u] >>= 8 * g;
            static_for<C::KS>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                const v4i a = lds_read_16(rbase + 16 * ((2 * s + g) ^ sw));
                const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
                const v8i b8 = {qf[s][0], qf[s][1], qf[s][2], qf[s][3], 0, 0, 0, 0};
                S[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, s == 0 ? v16f{} : S[kt], 4, 4,
                                                                        2 * (s % 2), int(kw[s / 2]), 0, qsc[s]);
            });
        }

        // ---- online softmax; key of lane half g, tile kt, register r: 32 g + 16 kt + r
        float mx = -INFINITY;
        if constexpr (MASK) {
            int lim = Nkv;
            if constexpr (CAUSAL) lim = min(lim, qidx + off + 1);
            int t = lim - j * kBlk - 32 * g;  // register (kt, r) visible iff 16 kt + r < t
            asm volatile("" : "+v"(t));
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (!(16 * kt + r < t)) S[kt][r] = -INFINITY;
        }
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            float a = max3f(S[kt][0], S[kt][1], S[kt][2]);
#pragma unroll
            for (int r = 3; r + 1 < 16; r += 2) a = max3f(a, S[kt][r], S[kt][r + 1]);
            mx = max3f(mx, a, S[kt][15]);
        }
        // the tile's row maximum in log2 units, rounded toward -inf, so that the fma
        // t = S c - m of the maximum is >= 0 and below one ulp of m: its p is 1
        float tr;
        {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            tr = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        float mt = tr * c;
        if (__builtin_fmaf(tr, c, -mt) < 0.0f) mt = __uint_as_float(__float_as_uint(mt) + (mt > 0.0f ? -1 : 1));
        const float mnew = __builtin_elementwise_maximum(m, mt);  // both finite or -inf
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        const int E = mx_exp_dev(__builtin_amdgcn_exp2f(__builtin_fmaf(mx, c, -mnew)));
        const float X = __uint_as_float(uint32_t(E + 127) << 23);
        v4i pk;
        float acc[4];
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const int kt = w >> 1, r0 = 8 * (w & 1);
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                q[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r0 + e], c, -mnew));
                acc[e & 3] = (w == 0 && e < 4) ? q[e] : acc[e & 3] + q[e];
            }
            // the first conversion writes byte 0; the other three overwrite the rest, so the
            // register's previous contents (q[1]'s, dead after it) do not matter
            int x = __float_as_int(q[1]);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[0], q[1], X, 0);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[2], q[3], X, 1);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[4], q[5], X, 2);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[6], q[7], X, 3);
            pk[w] = x;
        }
        l = __builtin_fmaf(l, alpha, (acc[0] + acc[1]) + (acc[2] + acc[3]));
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < C::DT; dt++) O[dt] *= alpha;
        }

        // ---- O^T += V^T P^T
        const v8i b8 = {pk[0], pk[1], pk[2], pk[3], 0, 0, 0, 0};
        const uint8_t* vst = st + C::KBYTES;
        // this lane's V exponents, byte dt for channel tile dt, picked by the byte select
        uint32_t vw[(C::NE + 3) / 4];
        load_exp_words<C::NE>(vex + (g * 32 + i) * C::NE, vw);
        static_for<C::DT>([&](auto dc) {
            constexpr int dt = decltype(dc)::value;
            const int d = 32 * dt + i;
            const v4i a = lds_read_16(vst + d * C::VROW + 16 * (g ^ mx_vswz(d)));
            const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
            O[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, O[dt], 4, 4, dt % 4, int(vw[dt / 4]), 0,
                                                                    E + 127);
        });
    };
    int j = 0;
    for (; j < jm; j++) step(std::false_type{}, j);
    for (; j < jend; j++) step(std::true_type{}, j);
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++) asm volatile("" : "+v"(O[dt]));

    // ---- epilogue: O^T / l -> out dtype, input layout
    if (!active) return;
    const float ltot = halves_sum(l);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;  // a query that sees no key: zeros
    if (qidx >= Nq) return;
    const bool vec4 = (p.D & 3) == 0;
    const int64_t obase = p.qm.cu != nullptr ? qv.start * p.osq : b * p.osb;
    uint16_t* orow = (uint16_t*)p.out + obase + h * p.osh + qidx * p.osq;
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
        for (int a4 = 0; a4 < 4; a4++) {
            const int d0 = 32 * dt + 8 * a4 + 4 * g;
            if (d0 >= p.D) continue;
            uint16_t hv[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float o = O[dt][4 * a4 + e] * inv;
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

template <int DP, bool CAUSAL, bool OBF16, bool QF>
hipError_t launch_mx_attn_t(const AttnMXArgs& a, hipStream_t s) {
    using C = MXCfg<DP>;
    MXParams p;
    p.q4 = a.q4;
    p.q4_exp = a.q4_exp;
    p.k4 = a.k4;
    p.k4_exp = a.k4_exp;
    p.v4 = a.v4;
    p.v4_exp = a.v4_exp;
    p.out = a.out;
    // the quantised operands' rows and slots (dense or packed)
    p.qm = make_seq_map(0, a.cu_q, a.B, a.Hq, a.Nq, a.total_q, a.D);
    p.km = make_seq_map(0, a.cu_k, a.B, a.Hkv, a.Nkv, a.total_k, a.D);
    const bool tok_major = a.out_nhd || a.cu_q != nullptr;  // (.., token, head, dim) output
    p.osb = a.cu_q != nullptr ? 0 : (a.out_nhd ? int64_t(a.Nq) * a.Hq * a.D : int64_t(a.Hq) * a.Nq * a.D);
    p.osh = tok_major ? int64_t(a.D) : int64_t(a.Nq) * a.D;
    p.osq = tok_major ? int64_t(a.Hq) * a.D : int64_t(a.D);
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.D = a.D;
    p.QT = (a.Nq + C::BM - 1) / C::BM;
    // K4 and V4 of one kv head: codes (DP / 2 bytes per token each) and exponents
    p.grp = causal_head_group(int64_t((a.Nkv + kBlk - 1) / kBlk) * kBlk * (DP + DP / 16),
                              int64_t(p.QT) * a.Hq * a.B, int64_t(p.G) * p.QT);
    p.cscale = a.sm_scale * 1.4426950408889634f;
    p.q16 = (const uint16_t*)a.q16;
    p.qst = make_strides(a.q_nhd, a.Hq, a.Nq, a.D);
    p.q_bf16 = a.q_bf16;
    p.q4_out = a.q4_out;
    p.q4_exp_out = a.q4_exp_out;
    const int64_t grid = int64_t(p.QT) * a.Hq * a.B;
    attn_mx_kernel<DP, CAUSAL, OBF16, QF><<<dim3(unsigned(grid)), C::THREADS, 0, s>>>(p);
    return hipGetLastError();
}

template <int DP, bool QF>
hipError_t launch_mx_attn_q(const AttnMXArgs& a, hipStream_t s) {
    if (a.causal)
        return a.out_bf16 ? launch_mx_attn_t<DP, true, true, QF>(a, s) : launch_mx_attn_t<DP, true, false, QF>(a, s);
    return a.out_bf16 ? launch_mx_attn_t<DP, false, true, QF>(a, s) : launch_mx_attn_t<DP, false, false, QF>(a, s);
}
template <int DP>
hipError_t launch_mx_attn_dp(const AttnMXArgs& a, hipStream_t s) {
    return a.q16 != nullptr ? launch_mx_attn_q<DP, true>(a, s) : launch_mx_attn_q<DP, false>(a, s);
}

}  // namespace

hipError_t launch_attn_mxfp4(const AttnMXArgs& a, hipStream_t s) {
    if (a.D <= 64) return launch_mx_attn_dp<64>(a, s);
    return a.D <= 128 ? launch_mx_attn_dp<128>(a, s) : launch_mx_attn_dp<256>(a, s);
}

}  // namespace sage
