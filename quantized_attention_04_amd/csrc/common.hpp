// common.hpp -- shared device helpers for the gfx950 kernels (internal header).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

constexpr int kBlk = 64;  // tokens per quantisation block and per KV tile
constexpr int kWave = 64;

// ---- where the tokens of one (batch entry, head) live -------------------------------
struct Strides {
    int64_t b, h, t;  // element strides of batch, head, token (channel stride is 1)
};

__host__ __device__ inline Strides make_strides(int layout_nhd, int H, int N, int D) {
    Strides s;
    if (layout_nhd) {
        s.b = int64_t(N) * H * D;
        s.h = D;
        s.t = int64_t(H) * D;
    } else {
        s.b = int64_t(H) * N * D;
        s.h = int64_t(N) * D;
        s.t = D;
    }
    return s;
}

// A batch of sequences, either dense (every sequence N tokens, input strides st) or
// packed (sequence b = tokens cu[b] .. cu[b+1]-1 of one axis of a (total, H, D)
// tensor).  Quantised rows and per-block slots: dense, (b, h) owns rows
// (b*H + h)*NB*64 .. and slots (b*H + h)*NB ..; packed, head h owns `rows` rows and
// `slots` slots and sequence b starts at row R_b = cu[b] + 64*b (slot floor(R_b/64)),
// which keeps every sequence's blocks disjoint without a prefix scan over the batch.
struct SeqMap {
    const int32_t* cu;   // packed: device prefix sums [B + 1]; dense: null
    Strides st;          // input strides (packed: t = H*D, h = D)
    int H, N, NB;        // heads; dense: tokens and 64-token blocks per sequence
    int total, maxlen;   // packed: tokens in all, bound on one sequence's length
    int64_t rows, slots; // packed: quantised rows and block slots per head
};
struct SeqView {
    int64_t start;   // first token on the input's token axis (packed), else 0
    int64_t in_off;  // element offset of (token 0, channel 0) of this (b, h) in the input
    int n;           // tokens
    int64_t row0;    // quantised row of token 0
    int64_t slot0;   // slot of block 0
};
// The map of a dense batch (cu == null: B sequences of `n` tokens, input layout HND
// or NHD) or of a packed one (cu != null: `n` bounds every sequence, `total` tokens in
// all, input (total, H, D)).  N and NB then give the grid extents.
inline SeqMap make_seq_map(int layout_nhd, const int32_t* cu, int B, int H, int n, int total, int D) {
    SeqMap m{};
    m.cu = cu;
    m.H = H;
    m.N = n;
    m.NB = (n + kBlk - 1) / kBlk;
    if (cu == nullptr) {
        m.st = make_strides(layout_nhd, H, n, D);
    } else {
        m.st = Strides{0, int64_t(D), int64_t(H) * D};
        m.total = total;
        m.maxlen = n;
        m.rows = int64_t(total) + int64_t(kBlk) * B;
        m.slots = (m.rows + kBlk - 1) / kBlk;
    }
    return m;
}

// Packed offsets are clamped into [0, total] and to maxlen, so inconsistent prefix
// sums give wrong numbers but never an access outside the tensors.
__device__ __forceinline__ SeqView seq_view(const SeqMap& m, int b, int h) {
    SeqView v;
    if (m.cu == nullptr) {
        v.start = 0;
        v.in_off = b * m.st.b + h * m.st.h;
        v.n = m.N;
        v.row0 = (int64_t(b) * m.H + h) * m.NB * kBlk;
        v.slot0 = (int64_t(b) * m.H + h) * m.NB;
    } else {
        const int s = min(max(m.cu[b], 0), m.total);
        const int e = min(max(m.cu[b + 1], s), m.total);
        v.n = min(e - s, m.maxlen);
        const int64_t R = int64_t(s) + int64_t(kBlk) * b;
        v.start = s;
        v.in_off = int64_t(s) * m.st.t + h * m.st.h;
        v.row0 = h * m.rows + R;
        v.slot0 = h * m.slots + R / kBlk;
    }
    return v;
}

// ---- element conversions -------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return float(h);
}
template <bool BF16>
__device__ __forceinline__ float in_to_f32(uint16_t b) {
    if constexpr (BF16) return bf16_bits_to_f32(b);
    else return f16_bits_to_f32(b);
}
// float -> bf16 bits, round half to even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

// ---- wave reductions --------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int parity(uint32_t x) { return __builtin_popcount(x) & 1; }

// Workgroup barrier without the memory fence of __syncthreads(): the fence would make
// the compiler wait for every outstanding global load, including the prefetch of the
// next tile.  LDS visibility is ensured by the explicit vmcnt waits before it; the
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Combine a value with the one held by the lane 32 positions away (the other half of
// the same query column): v_permlane32_swap returns the two halves side by side.
__device__ __forceinline__ float halves_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- waits --------------------------------------------------------------------------
// s_waitcnt vmcnt(n) with the other counters left at their maximum (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- direct global -> LDS copy of 16 bytes per lane ----------------------------------
// The LDS destination of lane i is lds_base + 16 * i (lds_base is wave-uniform).  Issued
// as inline asm: the instruction writes no VGPR, and keeping it opaque stops the
// compiler from guarding every later LDS read with a wait for ALL outstanding loads
// (it cannot tell a prefetch into one LDS stage from reads of the other).  Callers
// order it with explicit vmcnt waits and barriers.  Loads complete in issue order.
// The LDS base travels in M0 as a register operand of the statement (constraint
// "{m0}"), so the compiler loads M0 itself and knows the statement reads it.
__device__ __forceinline__ void load_lds_16(const void* gptr, void* lds_base) {
    const uint32_t lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds) : "memory");
}

// Same copy with the global address split into a wave-uniform 64-bit base (SGPR pair)
// and a per-lane 32-bit byte offset, and the LDS destination given as a wave-uniform
// LDS byte address plus a compile-time offset: no per-load 64-bit address arithmetic
// and a single live SGPR for the LDS side.
template <int LDS_OFF>
__device__ __forceinline__ void load_lds_16_s(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_wave_base + uint32_t(LDS_OFF))
                 : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ v4i lds_read_16(const void* p) { return *(const v4i*)p; }

// Scalar (SMEM) load of a wave-uniform float: counted by lgkmcnt, so it never waits on
// (or forces the completion of) outstanding vector-memory prefetches.
__device__ __forceinline__ float scalar_load_f32(const float* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const __attribute__((address_space(4))) float* c =
        (const __attribute__((address_space(4))) float*)(((uint64_t)hi << 32) | lo);
    return *c;
}

// XCD-aware remap: consecutive logical ids land on the same XCD (the hardware hands
// workgroup i to XCD i % 8), so workgroups that share K/V tiles share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    int xcd = bid % kXcd, idx = bid / kXcd;
    int per = nblocks / kXcd, rem = nblocks % kXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Workgroup -> (batch b, query head h, query tile qt) of a grid of B * Hkv * G * QT
// attention workgroups.  Consecutive logical ids on one XCD share a (b, kv head), so the
// K/V tiles they all stream come from that XCD's L2.  Causal: the query tiles of a group
// of grp kv heads run together in decreasing order of work (longest first), which
// shortens each group's tail while its K/V still fit in L2 and MALL; grp = 1 is plain
// head-by-head order.
// splits > 1 (key-range splits of one query tile): the splits of a query tile are
// consecutive logical ids, so they share the tile's Q rows and the head's K/V on one XCD;
// s returns the split index.
template <bool CAUSAL>
__device__ __forceinline__ void block_tile(int B, int Hkv, int G, int QT, int grp, int& b, int& h, int& qt,
                                           int splits = 1, int* s = nullptr) {
    int L = xcd_remap(blockIdx.x, gridDim.x);
    if (splits > 1) {
        *s = L % splits;
        L /= splits;
    }
    int bhk, hg;
    if constexpr (CAUSAL) {
        const int per = grp * G * QT, nkv = B * Hkv;
        const int gi = L / per, r = L % per;
        const int gsz = min(grp, nkv - gi * grp);  // the last group may be smaller
        hg = r % G;
        qt = QT - 1 - r / (G * gsz);
        bhk = gi * grp + (r / G) % gsz;
    } else {
        hg = L % G;
        qt = (L / G) % QT;
        bhk = L / (G * QT);
    }
    b = bhk / Hkv;
    h = (bhk % Hkv) * G + hg;
}

// Host: kv heads per causal group -- the largest power of two (up to 32) whose K and V
// operands (head_bytes each) fit 8 MiB together (an XCD's 4 MB L2 plus its share of the
// MALL).  Groups of more than four heads are taken only where their workgroups
// (wg_per_kv_head each) fit one XCD's share of the grid: the hardware hands workgroup i
// to XCD i % 8 and xcd_remap gives each XCD a contiguous range of logical ids, so such a
// group's longest-first order then spans every head on its XCD (short sequences: 1K
// causal 12% faster than with groups of four) instead of being cut across XCDs.
inline int causal_head_group(int64_t head_bytes, int64_t wg_total, int64_t wg_per_kv_head) {
    const int64_t budget = int64_t(8) << 20;
    const int64_t per_xcd = wg_total / 8;
    int grp = 1;
    for (int g = 2; g <= 32; g *= 2)
        if (g * head_bytes <= budget && (g <= 4 || g * wg_per_kv_head <= per_xcd)) grp = g;
    return grp;
}

}  // namespace sage
