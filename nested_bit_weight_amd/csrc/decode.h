// decode.h -- in-register decode of MSB-first bit-planes into bf16 MFMA/dot2
// operands, for gfx950.
//
// The r-bit child of a parent code keeps its top r bits (MatGPTQ: Accurate and
// Efficient Post-Training Matryoshka Quantization, abstract: slicing the most
// significant bits), and reads exactly r planes (MatGPTQ: Efficient and
// Accurate Inference over Nested Quantized Models, Abstract; Table 1, "Exact
// r-bit loading").  The kernels therefore receive, per 32 columns of one row,
// r 32-bit words P_0..P_{r-1} (P_0 = MSB plane) in the library layout: column
// e of the 32 sits at bit e/2 + 16*(e%2), so the column pair (2m, 2m+1) sits at
// bits (m, m+16) -- the two 16-bit halves of a bf16 pair.
//
// Decoding runs in two phases, both plain 32-bit VALU work:
//
//  1. A bit-matrix transpose network of delta swaps ("merge", below) turns up
//     to four plane words into words whose 1-, 2- or 4-bit fields each hold
//     one column's code, MSB first.  A merge of words a, b at distance d with
//     mask m is its own inverse, so the packer runs the same network backwards.
//
//  2. Each output word D_m (the bf16 pair of columns 2m, 2m+1) is cut out of a
//     network word with one shift and one and-or:
//         D_m = ((Z >> shift) & mask) | MAGIC
//     where MAGIC holds the bf16 exponent 2^E in both halves and the code lands
//     in the mantissa.  With the code's least significant bit at mantissa bit
//     `lsb`, the bf16 value is exactly 2^E + q * 2^(E - 7 + lsb).  E is chosen
//     per pair so that the coefficient of q is the same power of two for every
//     column; the per-column constant 2^E ("offset") is removed afterwards by
//     a correction that depends only on X (sum_k x_k * offset_k), computed
//     once per group and batch row and shared by every weight row.  All
//     operands are exact: q has at most 4 bits per phase, well inside bf16's
//     8-bit significand.
//
// Codes wider than 4 bits (r = 5..8) are decoded as two phases of at most 4
// planes: planes 0..3 (coefficient 2^(r-4)) and planes 4..r-1 (coefficient 1),
// whose products sum to the full code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nbw {

typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- network

// Delta swap: hi takes a's bits under m and b's bits (shifted down by d) under
// ~m; lo takes a's bits under ~m (shifted up by d) and b's bits under ~m.
__host__ __device__ __forceinline__ void merge(uint32_t a, uint32_t b, int d, uint32_t m, uint32_t &hi,
                                      uint32_t &lo) {
    hi = (a & m) | ((b >> d) & ~m);
    lo = ((a << d) & m) | (b & ~m);
}

constexpr uint32_t M1 = 0xAAAAAAAAu;
constexpr uint32_t M2 = 0xCCCCCCCCu;
constexpr uint32_t M4 = 0xF0F0F0F0u;

// Number of network words produced for RP planes (1..4).
template <int RP> struct NetWords { static constexpr int value = RP == 1 ? 1 : RP == 2 ? 2 : 4; };

// Phase 1 for RP planes (1..4).  Output word index w and field layout:
//  RP = 1: w0 = P0; bit b is column position b.
//  RP = 2: w0 = even positions, w1 = odd positions; field j (bits 2j..2j+1)
//          of w_t is the code of position 2j + t.
//  RP = 3, 4: w_s (s = 0..3); nibble j (bits 4j..4j+3) of w_s is the code of
//          position 4j + s (for RP = 3 the nibble is (code << 1)).
template <int RP>
__host__ __device__ __forceinline__ void network(const uint32_t *P, uint32_t *Z) {
    if constexpr (RP == 1) {
        Z[0] = P[0];
    } else if constexpr (RP == 2) {
        merge(P[0], P[1], 1, M1, Z[1], Z[0]);
    } else {
        uint32_t h01, l01, h23, l23;
        merge(P[0], P[1], 1, M1, h01, l01);
        if constexpr (RP == 4) {
            merge(P[2], P[3], 1, M1, h23, l23);
        } else {
            h23 = P[2] & M1;
            l23 = (P[2] << 1) & M1;
        }
        merge(h01, h23, 2, M2, Z[3], Z[1]);
        merge(l01, l23, 2, M2, Z[2], Z[0]);
    }
}

// ---------------------------------------------------------------- extraction plan

// For pair m (0..15) of an RP-plane phase: which network word, the right
// shift, and the bit of the code's LSB inside each 16-bit half after the shift.
struct Pick {
    int word, shift, lsb;
};

template <int RP> __host__ __device__ constexpr Pick pick(int m) {
    if (RP == 1) {
        int sh = m < 7 ? 0 : (m < 14 ? 7 : 14);
        return Pick{0, sh, m - sh};
    } else if (RP == 2) {
        int t = m & 1, j = m >> 1;
        int sh = j < 3 ? 0 : (j < 6 ? 6 : 12);
        return Pick{t, sh, 2 * j - sh};
    } else if (RP == 3) {
        // nibble j holds (code << 1): code bits 4j+1 .. 4j+3.  Nibbles 1 and 2
        // share one shift (by 5: bits 0..2 and 4..6), so a word takes two
        // shifts instead of three.
        int s = m & 3, j = m >> 2;
        int sh = j == 0 ? 0 : j == 3 ? 9 : 5;
        int lsb = j == 0 ? 1 : j == 1 ? 0 : 4;
        return Pick{s, sh, lsb};
    } else {
        int s = m & 3, j = m >> 2;
        int sh = j == 0 ? 0 : 4 * j - 3;
        int nib = j == 0 ? 0 : 3;      // nibble's bit 0 after the shift
        return Pick{s, sh, nib};
    }
}

template <int RP> __host__ __device__ constexpr uint32_t pick_mask(int m) {
    uint32_t f = ((1u << RP) - 1u) << pick<RP>(m).lsb;
    return f | (f << 16);
}

// bf16 exponent field value (biased) for pair m, code coefficient 2^C.
template <int RP, int C> __host__ __device__ constexpr uint32_t pick_expo(int m) {
    return (uint32_t)(127 + C + 7 - pick<RP>(m).lsb);
}

template <int RP, int C> __host__ __device__ constexpr uint32_t pick_magic(int m) {
    uint32_t h = pick_expo<RP, C>(m) << 7;
    return h | (h << 16);
}

// The constant part (offset) of pair m's bf16 values, as a bf16 pair bit
// pattern (offset = 2^(C + 7 - lsb), the magic with an all-zero code).
template <int RP, int C> __host__ __device__ constexpr uint32_t pick_offset_pair(int m) {
    return pick_magic<RP, C>(m);
}

// A constant held in a vector register.  gfx950 VALU instructions with three
// operands accept no literal constant and at most one scalar one, so
// `(z & mask) | magic` with both constants as literals costs two instructions
// (and + or); with them in VGPRs it is one v_and_or_b32.  The asm has no side
// effects, so the compiler hoists it out of loops like any constant.
__host__ __device__ __forceinline__ uint32_t vconst(uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
    return v;
#else
    return c;
#endif
}

// A constant held in a scalar register.  v_and_or_b32 reading the mask from
// an SGPR and the magic from a VGPR reads two VGPRs instead of three, which
// measured about 4.2 instead of 6 cycles per wave on gfx950.
__host__ __device__ __forceinline__ uint32_t sconst(uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t v;
    asm("s_mov_b32 %0, %1" : "=s"(v) : "i"(c));
    return v;
#else
    return c;
#endif
}

// Phase 2 for one pair.
template <int RP, int C>
__host__ __device__ __forceinline__ uint32_t extract(const uint32_t *Z, int m) {
    const Pick p = pick<RP>(m);
    uint32_t z = Z[p.word];
    if (p.shift) z >>= p.shift;
    return (z & sconst(pick_mask<RP>(m))) | vconst(pick_magic<RP, C>(m));
}

// Decode one 32-column word set of RP planes into 16 bf16 pairs (column pairs
// 2m, 2m+1 for m = 0..15), code coefficient 2^C.
template <int RP, int C>
__host__ __device__ __forceinline__ void decode_phase(const uint32_t *P, uint32_t *D) {
    uint32_t Z[NetWords<RP>::value];
    network<RP>(P, Z);
#pragma unroll
    for (int m = 0; m < 16; ++m) D[m] = extract<RP, C>(Z, m);
}

// Number of phases for an r-bit child and the planes in each.
template <int R> struct Phases {
    static constexpr int count = R <= 4 ? 1 : 2;
    static constexpr int rp0 = R <= 4 ? R : 4;   // planes 0..rp0-1
    static constexpr int rp1 = R <= 4 ? 0 : R - 4; // planes 4..R-1
    static constexpr int c0 = R <= 4 ? 0 : R - 4; // coefficient exponent of phase 0
};

// Offset classes: the decoded operand of pair m is offset_m + coefficient*q,
// with offset_m = 2^(C + 7 - lsb_m) per phase, so it depends on m only
// through (lsb of phase 0, lsb of phase 1) -- a handful of classes.  The
// correction sum_k x_k * (1/2 - 2^(R-1) - offset_k) therefore needs the pair
// sums (x_lo + x_hi) collected per class (one dot2 per pair) and one FMA per
// class, not a product per column.
template <int R> __host__ __device__ constexpr int lsb0(int m) { return pick<Phases<R>::rp0>(m).lsb; }
template <int R> __host__ __device__ constexpr int lsb1(int m) {
    return Phases<R>::rp1 > 0 ? pick<(Phases<R>::rp1 > 0 ? Phases<R>::rp1 : 1)>(m).lsb : 0;
}
template <int R> __host__ __device__ constexpr bool class_used(int a, int b) {
    for (int m = 0; m < 16; ++m)
        if (lsb0<R>(m) == a && lsb1<R>(m) == b) return true;
    return false;
}

// Coefficient of the pair sum (x_2m + x_2m+1) in the correction of pair m:
// the exact operand is q + 1/2 - 2^(R-1), the decoded one offset_m + q.
template <int R> __host__ __device__ constexpr float pair_coef(int m) {
    float off = (float)(1u << (Phases<R>::c0 + 7 - lsb0<R>(m)));
    if (Phases<R>::rp1 > 0) off += (float)(1u << (7 - lsb1<R>(m)));
    return 0.5f - (float)(1 << (R - 1)) - off;
}

// Correction for NP bf16 pairs (a multiple of 16, pair index mod 16 = m).
template <int R, int NP>
__device__ __forceinline__ float correction(const uint32_t *X2) {
    constexpr int c0 = Phases<R>::c0;
    float cls[7][7];
#pragma unroll
    for (int a = 0; a < 7; ++a)
#pragma unroll
        for (int b = 0; b < 7; ++b) cls[a][b] = 0.f;
    const uint32_t one = 0x3F803F80u;  // bf16 (1.0, 1.0)
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const int m = q & 15;
        float &c = cls[lsb0<R>(m)][lsb1<R>(m)];
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, one),
                                            __builtin_bit_cast(bf16x2_t, X2[q]), c, false);
    }
    float corr = 0.f;
#pragma unroll
    for (int a = 0; a < 7; ++a)
#pragma unroll
        for (int b = 0; b < 7; ++b)
            if (class_used<R>(a, b)) {
                float off = (float)(1u << (c0 + 7 - a));
                if constexpr (Phases<R>::rp1 > 0) off += (float)(1u << (7 - b));
                const float coef = 0.5f - (float)(1 << (R - 1)) - off;
                corr = fmaf(coef, cls[a][b], corr);
            }
    return corr;
}

// Decode the r-bit codes of one word set into D0 (phase 0) and D1 (phase 1,
// R > 4 only).  P: R plane words, P[p] = plane p.
template <int R>
__host__ __device__ __forceinline__ void decode_word(const uint32_t *P, uint32_t *D0, uint32_t *D1) {
    decode_phase<Phases<R>::rp0, Phases<R>::c0>(P, D0);
    if constexpr (Phases<R>::count == 2) decode_phase<Phases<R>::rp1, 0>(P + 4, D1);
}

// Single-phase decode for R = 5..8 (the large-batch GEMM): each column's
// child code as one bf16 integer, q * 2^(8-R) (at most 8 significant bits,
// so exact; the two-phase decode above needs two MFMA operands per column).
// Planes 0..3 and 4..7 (those at or past R read as zero) go through the
// four-plane network; one byte-level merge per word then joins the two
// nibbles of each position into its code byte (high nibble from planes
// 0..3), and byte k of a word converts to fp32 exactly, whose top half is
// the bf16 value.  Output D[m] = bf16 pair (column 2m, column 2m+1), i.e.
// positions m and m + 16 of the plane words.
// bf16 pair (lo, hi) from two fp32 values whose low 16 bits are zero: the
// top halves of their bit patterns.
__host__ __device__ __forceinline__ uint32_t pair_of_f32_tops(float lo, float hi) {
    const uint32_t l = __builtin_bit_cast(uint32_t, lo), h = __builtin_bit_cast(uint32_t, hi);
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(h, l, 0x07060302u);
#else
    return (h & 0xFFFF0000u) | (l >> 16);
#endif
}

template <int R>
__host__ __device__ __forceinline__ void decode_word_bytes(const uint32_t *P, uint32_t *D) {
    static_assert(R >= 5 && R <= 8, "byte decode is for 5..8 planes");
    uint32_t Ph[4] = {P[0], P[1], P[2], P[3]};
    uint32_t Pl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) Pl[p] = 4 + p < R ? P[4 + p] : 0u;
    uint32_t Zh[4], Zl[4];
    network<4>(Ph, Zh);
    network<4>(Pl, Zl);
    // BH[s] byte k: code of position 4(2k+1) + s; BL[s] byte k: position 8k + s.
    uint32_t BH[4], BL[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) merge(Zh[s], Zl[s], 4, M4, BH[s], BL[s]);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int s = m & 3, j = m >> 2;  // position m: nibble j of word s; m + 16: nibble j + 4
        const uint32_t wlo = (j & 1) ? BH[s] : BL[s];
        const int blo = (j & 1) ? (j - 1) >> 1 : j >> 1;
        const uint32_t whi = (j & 1) ? BH[s] : BL[s];
        const int bhi = (j & 1) ? (j + 3) >> 1 : (j + 4) >> 1;
        const float flo = (float)((wlo >> (8 * blo)) & 0xFFu);
        const float fhi = (float)((whi >> (8 * bhi)) & 0xFFu);
        D[m] = pair_of_f32_tops(flo, fhi);
    }
}

// Raw codes (no bf16) of pair m for an RP-plane phase: low half and high half.
template <int RP>
__host__ __device__ __forceinline__ uint32_t extract_codes(const uint32_t *Z, int m) {
    const Pick p = pick<RP>(m);
    uint32_t z = Z[p.word];
    if (p.shift) z >>= p.shift;
    z = (z & pick_mask<RP>(m)) >> p.lsb;
    return z;  // code(2m) in bits 0..RP-1, code(2m+1) in bits 16..16+RP-1
}

// ---------------------------------------------------------------- packing

// Byte `b` (0..3) of w.
__host__ __device__ __forceinline__ uint32_t byte_of(uint32_t w, int b) { return (w >> (8 * b)) & 0xFFu; }

// 32 codes (8 words, word q = columns 4q..4q+3) -> 8 plane words.
__host__ __device__ __forceinline__ void pack_word32(const uint32_t *W, uint32_t *P) {
    // Y_t: byte j holds the code at plane-bit position 8j + t, i.e. columns
    // 2t (j=0), 16+2t (j=1), 2t+1 (j=2), 17+2t (j=3).
    uint32_t Y[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t a = W[t >> 1], c = W[4 + (t >> 1)];
        const int b0 = 2 * (t & 1);
        Y[t] = byte_of(a, b0) | (byte_of(c, b0) << 8) | (byte_of(a, b0 + 1) << 16) |
               (byte_of(c, b0 + 1) << 24);
    }
    // Undo the byte-level merge: (B_hi = Y[4+s], B_lo = Y[s]) -> (Z_s, Z'_s).
    uint32_t Z[4], Zp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) merge(Y[4 + s], Y[s], 4, M4, Z[s], Zp[s]);
    // Undo the nibble-level merges.
    uint32_t h01, h23, l01, l23, h45, h67, l45, l67;
    merge(Z[3], Z[1], 2, M2, h01, h23);
    merge(Z[2], Z[0], 2, M2, l01, l23);
    merge(Zp[3], Zp[1], 2, M2, h45, h67);
    merge(Zp[2], Zp[0], 2, M2, l45, l67);
    // Undo the pair-level merges.
    merge(h01, l01, 1, M1, P[0], P[1]);
    merge(h23, l23, 1, M1, P[2], P[3]);
    merge(h45, l45, 1, M1, P[4], P[5]);
    merge(h67, l67, 1, M1, P[6], P[7]);
}

}  // namespace nbw
