// gfx950 kernels for the DeltaNet chunkwise-parallel forward pass.
//
// One workgroup (4 waves) owns a 64-row tile of one unit's state and walks
// that unit's chunks in order. Per chunk it runs the per-chunk algorithm of
// "Linear Attention, Visualized" (Haoran Zhang), DeltaNet > "Complete
// per-chunk algorithm", with the state transposed ("Context Parallelism for
// DeltaNet", yywangcs, section 2: S is dv x dk):
//   A  Gram and masked scores: A = diag(beta) (K K^T) strictly lower (fp32,
//      the matrix of the triangular solve) and P = (Q K^T) lower-inclusive
//   B  diagonal 16x16 blocks of N = (I + A)^-1 by forward substitution, one
//      column per lane, entries of A broadcast across the lane row with DPP
//      ("Solving for U": unit lower triangular, solved row after row)
//   C  off-diagonal blocks of N by block forward substitution on the matrix
//      cores; T = N diag(beta) solves (I + diag(beta) L) T = diag(beta)
//   D  W = T K (shared, stored as -W) and U = T V (per wave, in registers)
//   E  the chain: Z = U - W S^T, O = Q S^T + P Z, S <- S + Z^T K
// Rows of S are independent (row j of S, Z, U and O needs only row j and the
// shared K, Q, W), so each wave owns 16 state rows and runs E on its own;
// only A-D are shared through LDS.
//
// Gated DeltaNet (same page, "Gated DeltaNet (GDN)" > "Complete per-chunk
// algorithm"): with gamma_l the decay logarithms summed over the chunk up to
// token l, the masks of A and P take the factor exp(gamma_l - gamma_i), W is
// built from K with rows scaled by exp(gamma_l), the Q S^T part of O is
// scaled by exp(gamma_l) per token, and the update becomes
// S <- exp(gamma_C) S + Z^T (K with rows scaled by exp(gamma_C - gamma_l)).
// Every factor is a difference of two prefix sums with the later one first,
// so it lies in (0, 1]; pairs outside a mask are never multiplied in. The
// prefix sums are kept in LDS in base-2 units (times log2 e).
//
// This file holds the fp32 path: chain_kernel_serial (four waves, A-E one
// after the other; fp32 operands do not fit two chunks in LDS) and the
// context-parallel prefix composition. The bf16 path, with specialised waves
// and a different order of products, is chain_bf16.hip.
//
// Matrix-core layout facts used throughout (16x16 tiles, wave64, lane
// l = 16*g + c with g = l/16, c = l%16):
//   accumulator register i of lane l holds D[4g + i][c];
//   a "k16 fragment" is 4 consecutive k values 4g..4g+3 of a 16-deep k block
//   for row c (A operand) or column c (B operand).
// An accumulator tile therefore IS a k16 fragment for a product that
// contracts over the tile's rows, with its column index as the operand's free
// index -- so S, Z and the N blocks feed the next product straight from
// registers. A 16x16x32 bf16 product takes two k16 fragments (k blocks 2s and
// 2s+1); since A and B use the same pairing of (lane, value) to k, any
// consistent order of k inside the instruction is exact.
//
// Fragments are read from LDS in two ways. A "row" fragment (4 consecutive
// elements of one row) is one 8-byte read. A "column" fragment (4 consecutive
// rows of one column) of a row-major 16-bit matrix comes from the gfx950
// transposing read ds_read_b64_tr_b16: inside each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks supplied by lanes i/4 + 4e
// (e = 0..3), so lane p supplies row 4g + p/4, columns 4(p%4)..+3 and lane c
// receives column c, rows 4g..4g+3. K and V therefore stay row-major in LDS,
// and T is kept transposed so that every write of T is a vector store.
#include "dn_internal.h"
#include "dn_work.h"

namespace dn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <typename E> struct Tr;

// bf16 operands, fp32 accumulation.
template <> struct Tr<__bf16> {
    using F = bf16x4; // k16 fragment
    using V = bf16x8; // 16-byte vector
    static constexpr int kVec = 8;
    __device__ static inline f32x4 mma16(f32x4 c, F a, F b) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 mma32(f32x4 c, F a0, F a1, F b0, F b1) {
        const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Two packed conversions (round to nearest even). Written per pair and
    // reassembled through 32-bit words: element-wise conversion that feeds a
    // matrix-core operand is otherwise emitted as four single conversions
    // plus two permutes.
    __device__ static inline F cvt(f32x4 x) {
        const bf16x2 lo = __builtin_convertvector(__builtin_shufflevector(x, x, 0, 1), bf16x2);
        const bf16x2 hi = __builtin_convertvector(__builtin_shufflevector(x, x, 2, 3), bf16x2);
        const u32x2 u = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
        return __builtin_bit_cast(F, u);
    }
    __device__ static inline float tof(__bf16 x) { return (float)x; }
    __device__ static inline __bf16 fromf(float x) { return (__bf16)x; }
    __device__ static inline F scale(F x, f32x4 s) {
        const f32x4 w = {(float)x[0] * s[0], (float)x[1] * s[1], (float)x[2] * s[2], (float)x[3] * s[3]};
        return cvt(w);
    }
    // Y[k0 + 4g + e][n0 + c], e = 0..3, from a row-major LDS matrix (ld elements).
    __device__ static inline F ldcol(const __bf16 *Y, int ld, int k0, int n0, int g, int c) {
        const __bf16 *p = Y + (k0 + 4 * g + (c >> 2)) * ld + n0 + 4 * (c & 3);
        return __builtin_bit_cast(F, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
    }
};

// fp32 operands: four 16x16x4 products per k16 fragment. Product j takes
// value j of every lane group, i.e. k = 4g + j, so the four together cover the
// 16-deep block once. Column fragments are four scalar reads.
template <> struct Tr<float> {
    using F = f32x4;
    using V = f32x4;
    static constexpr int kVec = 4;
    __device__ static inline f32x4 mma16(f32x4 c, F a, F b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    __device__ static inline f32x4 mma32(f32x4 c, F a0, F a1, F b0, F b1) {
        return mma16(mma16(c, a0, b0), a1, b1);
    }
    __device__ static inline F cvt(f32x4 x) { return x; }
    __device__ static inline float tof(float x) { return x; }
    __device__ static inline float fromf(float x) { return x; }
    __device__ static inline F scale(F x, f32x4 s) { return x * s; }
    __device__ static inline F ldcol(const float *Y, int ld, int k0, int n0, int g, int c) {
        const float *p = Y + (k0 + 4 * g) * ld + n0 + c;
        F r = {p[0], p[ld], p[2 * ld], p[3 * ld]};
        return r;
    }
};

template <typename E> __device__ inline typename Tr<E>::F ldrow(const E *Y, int ld, int row, int k0, int g) {
    return *reinterpret_cast<const typename Tr<E>::F *>(Y + row * ld + k0 + 4 * g);
}
template <typename E> __device__ inline void stf(E *p, typename Tr<E>::F x) {
    *reinterpret_cast<typename Tr<E>::F *>(p) = x;
}

// Broadcast lane I of each 16-lane row to the whole row (DPP row_newbcast).
template <int I> __device__ inline float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + I,
                                                              0xF, 0xF, true));
}

// exp2 of each element (decay factors from base-2 prefix sums).
__device__ inline f32x4 exp2v(f32x4 x) {
    return f32x4{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]), __builtin_amdgcn_exp2f(x[2]),
                 __builtin_amdgcn_exp2f(x[3])};
}

// One column of (I + A)^-1 for a 16x16 strictly lower A held by rows (lane
// c16 of each 16-lane row holds row c16 of A): right-looking substitution,
// once x_J is final it is removed from every row below it.
template <int J> __device__ inline void solve_step(float (&x)[16], const float (&arow)[16]) {
    if constexpr (J < 15) {
        const float nxj = -x[J];
#define DN_UPD(I)                                                                                              \
    if constexpr (I > J) x[I] = fmaf(row_bcast<I>(arow[J]), nxj, x[I]);
        DN_UPD(1) DN_UPD(2) DN_UPD(3) DN_UPD(4) DN_UPD(5) DN_UPD(6) DN_UPD(7) DN_UPD(8)
        DN_UPD(9) DN_UPD(10) DN_UPD(11) DN_UPD(12) DN_UPD(13) DN_UPD(14) DN_UPD(15)
#undef DN_UPD
        solve_step<J + 1>(x, arow);
    }
}

// Row strides (elements), padded beyond a multiple of 128 elements so that
// the 16 rows touched by one fragment read spread over the LDS banks.
template <typename E, int DK> struct Ld {
    // rows padded by 8 elements: for bf16 a K row is 68 dwords and a 64-wide
    // row 36, so the 8-byte row reads of 16 rows at once fill all 64 banks
    // (a 16-element pad put rows r and r + 8 on the same banks; the gated
    // backward ran 4.5% faster with 8)
    static constexpr int kPadE = 8;
    static constexpr int K = DK + kPadE;     // K, Q, W: [C][K]
    static constexpr int V = kRows + kPadE;  // V tile: [C][V]
    static constexpr int T = kChunk + kPadE; // T^T, P: [C][T]
    static constexpr int A = kChunk + 4;     // A (fp32): [C][A]
    static constexpr int N = 16 + kPadE;     // N^T, 4 diagonal blocks: [64][N]
    static constexpr size_t szK = sizeof(E) * kChunk * K;
    static constexpr size_t szV = sizeof(E) * kChunk * V;
    static constexpr size_t szT = sizeof(E) * kChunk * T;
    static constexpr size_t szA = sizeof(float) * kChunk * A;
    static constexpr size_t szN = sizeof(E) * 64 * N;
    static constexpr size_t szWA = szA > szK ? szA : szK; // W and A share space
};

// The per-chunk phases, shared by both kernels. Each is executed by every
// wave (w = wave, g = lane group, c16 = lane in group) on LDS operands.
//
// Every phase is split into a fetch (all LDS operand fragments of the phase
// into registers) and a compute step. The kernels put a scheduling fence
// between the fetches and the computes of a barrier interval: all reads of
// the interval are in flight before the first matrix product needs one, so
// LDS latency is paid once per interval instead of once per product (with one
// wave per SIMD nothing else would hide it).
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <typename E, int DK> struct Phases {
    using TR = Tr<E>;
    using F = typename TR::F;
    using L = Ld<E, DK>;
    static constexpr int NMT = DK / 16; // 16-wide dk tiles
    static constexpr int NKB = DK / 32; // 32-deep k blocks over dk

    // ---- A: Gram (as the solve's A = beta_i k_i.k_j, j < i, fp32) and masked
    // scores P. Wave roles: 0 Gram rows {0,3}, 1 scores rows {0,3}, 2 Gram
    // rows {1,2}, 3 scores rows {1,2}; tile (a, c <= a) = K_c X_a^T with X = K
    // (Gram) or Q (scores). The role is a template argument so each wave's code
    // is free of branches.
    template <int W> struct GramFrags {
        static constexpr int A1 = (W < 2) ? 0 : 1, A2 = (W < 2) ? 3 : 2;
        F xb[2][NKB][2]; // X rows of blocks A1, A2
        F kc[A2 + 1][NKB][2]; // K rows of blocks 0..A2
    };
    template <int W>
    __device__ static inline void gram_fetch(GramFrags<W> &f, const E *Ks, const E *Qs, int g, int c16) {
        using G = GramFrags<W>;
        const E *X = (W & 1) ? Qs : Ks;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                f.xb[0][kb][h2] = ldrow(X, L::K, 16 * G::A1 + c16, 32 * kb + 16 * h2, g);
                f.xb[1][kb][h2] = ldrow(X, L::K, 16 * G::A2 + c16, 32 * kb + 16 * h2, g);
#pragma unroll
                for (int cb = 0; cb <= G::A2; ++cb)
                    f.kc[cb][kb][h2] = ldrow(Ks, L::K, 16 * cb + c16, 32 * kb + 16 * h2, g);
            }
    }
    template <int W, bool GATED>
    __device__ static inline void gram_compute(const GramFrags<W> &f, const float *Bs, const float *Gs, float *As,
                                               E *Ps, int g, int c16) {
        using G = GramFrags<W>;
        constexpr bool isP = W & 1;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const int ab = which ? G::A2 : G::A1;
#pragma unroll
            for (int cb = 0; cb <= G::A2; ++cb) {
                if (cb > ab) continue;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    acc = TR::mma32(acc, f.kc[cb][kb][0], f.kc[cb][kb][1], f.xb[which][kb][0], f.xb[which][kb][1]);
                // acc[e] = k_{16cb+4g+e} . x_{16ab+c16}
                const int row = 16 * ab + c16, col = 16 * cb + 4 * g;
                if constexpr (GATED) {
                    // decay between column token col + e and row token row (masked pairs unused)
                    const f32x4 gc = *reinterpret_cast<const f32x4 *>(Gs + col);
                    acc *= exp2v(Gs[row] - gc);
                }
                if constexpr (!isP) {
                    const float br = Bs[row];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = (col + e < row) ? acc[e] * br : 0.f;
                    *reinterpret_cast<f32x4 *>(As + row * L::A + col) = acc;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = (col + e > row) ? 0.f : acc[e];
                    stf(Ps + row * L::T + col, TR::cvt(acc));
                }
            }
        }
    }

    // ---- B: N_ww = (I + A_ww)^-1 for the diagonal block w, column c16 per
    // lane (all four lane groups compute the same column). Writes N_ww^T and
    // the diagonal block of T^T; returns N_ww as a k16 B fragment.
    struct DiagFrags {
        float arow[16]; // A[16w + c16][16w + j]
        float bc;       // beta_{16w + c16}
    };
    __device__ static inline void diag_fetch(DiagFrags &f, const float *As, const float *Bs, int w, int c16) {
        const int o = 16 * w;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(As + (o + c16) * L::A + o + 4 * j4);
            f.arow[4 * j4 + 0] = t[0];
            f.arow[4 * j4 + 1] = t[1];
            f.arow[4 * j4 + 2] = t[2];
            f.arow[4 * j4 + 3] = t[3];
        }
        f.bc = Bs[o + c16];
    }
    __device__ static inline F diag_compute(const DiagFrags &f, E *NsT, E *TsT, int w, int g, int c16) {
        const int o = 16 * w;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c16) ? 1.f : 0.f;
        solve_step<0>(x, f.arow);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 xv = {x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
            // every lane group writes the same values: no branch needed
            stf(NsT + (o + c16) * L::N + 4 * i4, TR::cvt(xv));
            stf(TsT + (o + c16) * L::T + o + 4 * i4, TR::cvt(xv * f.bc));
        }
        f32x4 xf;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xf[i] = g == 0 ? x[i] : g == 1 ? x[4 + i] : g == 2 ? x[8 + i] : x[12 + i];
        return TR::cvt(xf);
    }

    // ---- C: off-diagonal blocks of column block b of N:
    //   N_ab = -N_aa * sum_{c=b}^{a-1} A_ac N_cb,  a = b+1..3,  T_ab = N_ab diag(beta_b).
    template <int b> struct OffFrags {
        F arow[4][4]; // A_ac rows (a > b, b <= c < a)
        F nrow[4];    // rows of N_aa (a > b)
        float beta_col;
    };
    template <int b>
    __device__ static inline void off_fetch(OffFrags<b> &f, const float *As, const E *NsT, const float *Bs, int g,
                                            int c16) {
        f.beta_col = Bs[16 * b + c16];
#pragma unroll
        for (int a = b + 1; a < 4; ++a) {
#pragma unroll
            for (int c = b; c < a; ++c)
                f.arow[a][c] =
                    TR::cvt(*reinterpret_cast<const f32x4 *>(As + (16 * a + c16) * L::A + 16 * c + 4 * g));
            f.nrow[a] = TR::ldcol(NsT + a * 16 * L::N, L::N, 0, 0, g, c16); // row c16 of N_aa
        }
    }
    template <int b>
    __device__ static inline void off_compute(const OffFrags<b> &f, F nbb, E *TsT, int g, int c16) {
        F frag[4];
        frag[b] = nbb;
#pragma unroll
        for (int a = b + 1; a < 4; ++a) {
            f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = b; c < a; ++c) R = TR::mma16(R, f.arow[a][c], frag[c]);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 nab = -TR::mma16(z, f.nrow[a], TR::cvt(R));
            frag[a] = TR::cvt(nab);
            // nab[e] = N[16a + 4g + e][16b + c16] -> T^T row 16b + c16, columns 16a + 4g..
            stf(TsT + (16 * b + c16) * L::T + 16 * a + 4 * g, TR::cvt(nab * f.beta_col));
        }
    }

    // ---- D: -W = -(T K) for this wave's dk tiles to LDS; U = T V for this
    // wave's 16 value rows (zero when there is no V).
    struct WUFrags {
        F trow[4][4];        // T[16n + c16][16kk + 4g..] (kk <= n | 1)
        F kcol[NMT / 4][4];  // K[16kk + 4g..][16m + c16] for this wave's dk tiles m
        F vcol[4];           // V[16kk + 4g..][16w + c16]
    };
    template <bool GATED>
    __device__ static inline void wu_fetch(WUFrags &f, const E *Ks, const E *Vs, const E *TsT, const float *Gs,
                                           bool has_v, int w, int g, int c16) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                if (kk <= (n | 1)) f.trow[n][kk] = TR::ldcol(TsT, L::T, 16 * kk, 16 * n, g, c16);
#pragma unroll
        for (int mm = 0; mm < NMT / 4; ++mm)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                f.kcol[mm][kk] = TR::ldcol(Ks, L::K, 16 * kk, 16 * (w * (NMT / 4) + mm), g, c16);
                // W = T (K with token rows scaled by exp(gamma_l))
                if constexpr (GATED)
                    f.kcol[mm][kk] =
                        TR::scale(f.kcol[mm][kk], exp2v(*reinterpret_cast<const f32x4 *>(Gs + 16 * kk + 4 * g)));
            }
        if (has_v) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.vcol[kk] = TR::ldcol(Vs, L::V, 16 * kk, 16 * w, g, c16);
        }
    }
    __device__ static inline void wu_compute(const WUFrags &f, E *Ws, bool has_v, f32x4 (&Zacc)[4], int w, int g,
                                             int c16) {
#pragma unroll
        for (int mm = 0; mm < NMT / 4; ++mm) {
            const int m = w * (NMT / 4) + mm;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= n / 2; ++s)
                    acc = TR::mma32(acc, f.kcol[mm][2 * s], f.kcol[mm][2 * s + 1], f.trow[n][2 * s],
                                    f.trow[n][2 * s + 1]);
                // acc[e] = W[16n + c16][16m + 4g + e]
                stf(Ws + (16 * n + c16) * L::K + 16 * m + 4 * g, TR::cvt(-acc));
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (has_v) {
#pragma unroll
                for (int s = 0; s <= t / 2; ++s)
                    acc = TR::mma32(acc, f.trow[t][2 * s], f.trow[t][2 * s + 1], f.vcol[2 * s], f.vcol[2 * s + 1]);
            }
            Zacc[t] = acc; // U[16t + 4g + e][row 16w + c16]
        }
    }

    // ---- E1: Z = U - W S^T (Ws holds -W); result as k16 fragments over tokens.
    struct ZFrags {
        F wr[4][NKB][2]; // -W rows 16t + c16
    };
    __device__ static inline void z_fetch(ZFrags &f, const E *Ws, int g, int c16) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                f.wr[t][kb][0] = ldrow(Ws, L::K, 16 * t + c16, 32 * kb, g);
                f.wr[t][kb][1] = ldrow(Ws, L::K, 16 * t + c16, 32 * kb + 16, g);
            }
    }
    __device__ static inline void z_compute(const ZFrags &f, const F (&SB)[NMT], const f32x4 (&Zacc)[4], F (&ZB)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 z = Zacc[t];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) z = TR::mma32(z, f.wr[t][kb][0], f.wr[t][kb][1], SB[2 * kb], SB[2 * kb + 1]);
            ZB[t] = TR::cvt(z); // Z[16t + 4g + e][row 16w + c16]
        }
    }

    // ---- E2: O^T tiles = S Q^T + Z^T P^T (with the pre-update S);
    // Oacc[t][e] = O[16t + c16][16w + 4g + e].
    struct OFrags {
        F qr[4][NKB][2]; // Q rows 16t + c16
        F pr[4][2][2];   // P rows 16t + c16, k blocks s <= t/2
        float eq[4];     // exp(gamma) of token 16t + c16 (gated)
    };
    template <bool GATED>
    __device__ static inline void o_fetch(OFrags &f, const E *Qs, const E *Ps, const float *Gs, int g, int c16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                f.qr[t][kb][0] = ldrow(Qs, L::K, 16 * t + c16, 32 * kb, g);
                f.qr[t][kb][1] = ldrow(Qs, L::K, 16 * t + c16, 32 * kb + 16, g);
            }
#pragma unroll
            for (int s = 0; s <= t / 2; ++s) {
                f.pr[t][s][0] = ldrow(Ps, L::T, 16 * t + c16, 32 * s, g);
                f.pr[t][s][1] = ldrow(Ps, L::T, 16 * t + c16, 32 * s + 16, g);
            }
            if constexpr (GATED) f.eq[t] = __builtin_amdgcn_exp2f(Gs[16 * t + c16]);
        }
    }
    template <bool GATED>
    __device__ static inline void o_compute(const OFrags &f, const F (&SB)[NMT], const F (&ZB)[4], f32x4 (&Oacc)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) acc = TR::mma32(acc, SB[2 * kb], SB[2 * kb + 1], f.qr[t][kb][0], f.qr[t][kb][1]);
            if constexpr (GATED) acc *= f.eq[t]; // Q rows scaled by exp(gamma_l)
#pragma unroll
            for (int s = 0; s <= t / 2; ++s) acc = TR::mma32(acc, ZB[2 * s], ZB[2 * s + 1], f.pr[t][s][0], f.pr[t][s][1]);
            Oacc[t] = acc;
        }
    }

    // ---- E3: S^T += K^T Z (gated: S^T <- exp(gamma_C) S^T + (K rows scaled by
    // exp(gamma_C - gamma_l))^T Z).
    struct SFrags {
        F kc[NMT][4]; // K[16kk + 4g..][16m + c16]
        float ec;     // exp(gamma_C) (gated)
    };
    template <bool GATED> __device__ static inline void s_fetch(SFrags &f, const E *Ks, const float *Gs, int g, int c16) {
        f32x4 er[4];
        if constexpr (GATED) {
            const float gC = Gs[kChunk - 1];
            f.ec = __builtin_amdgcn_exp2f(gC);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) er[kk] = exp2v(gC - *reinterpret_cast<const f32x4 *>(Gs + 16 * kk + 4 * g));
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                f.kc[m][kk] = TR::ldcol(Ks, L::K, 16 * kk, 16 * m, g, c16);
                if constexpr (GATED) f.kc[m][kk] = TR::scale(f.kc[m][kk], er[kk]);
            }
    }
    template <bool GATED>
    __device__ static inline void s_compute(const SFrags &f, const F (&ZB)[4], f32x4 (&Sacc)[NMT]) {
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            if constexpr (GATED) Sacc[m] *= f.ec;
            Sacc[m] = TR::mma32(Sacc[m], f.kc[m][0], f.kc[m][1], ZB[0], ZB[1]);
            Sacc[m] = TR::mma32(Sacc[m], f.kc[m][2], f.kc[m][3], ZB[2], ZB[3]);
        }
    }
};

// Global -> register -> LDS staging of one chunk (K, Q, V tile, beta).
// Loads are unconditional: rows past the end of the sequence re-read the last
// valid row (always in bounds) and become zeros when written to LDS, so no
// load sits behind a branch; beta stays raw until it is written.
template <typename E, int DK, int NT = kThreads> struct Stager {
    using TR = Tr<E>;
    using V = typename TR::V;
    using L = Ld<E, DK>;
    static constexpr int KQV = DK / TR::kVec;           // vectors per K/Q row
    static constexpr int NKQ = kChunk * KQV / NT;       // K (and Q) vectors per thread
    static constexpr int VV = kRows / TR::kVec;         // vectors per V-tile row
    static constexpr int NVV = kChunk * VV / NT;        // V vectors per thread
    static_assert(NKQ * NT == kChunk * KQV && NVV * NT == kChunk * VV, "tiling");

    const E *kg, *qg, *vg, *bg;
    const float *gg; // log decays, or nullptr
    // Gated path: queries and decays are addressed by real token (virtual
    // step tok0 + row is substep (.) % nh of real token (.) / nh); qh and gh
    // point at this head's real token 0.
    const E *qh;
    const float *gh;
    SubstepBase sb;
    int64_t sqk, sv;
    int H, len, tid;
    bool has_v;
    V rk[NKQ], rq[NKQ], rv[NVV];
    E rbeta;
    float rg;
    // gated: whether the loaded query (decay) belongs to this substep; applied
    // at staging so that no select waits on a load in flight
    bool qon[NKQ], gon;
    int nval;

    __device__ inline void load(int c) {
        nval = min(kChunk, len - c * kChunk);
        const int last = nval - 1;
        const int64_t base = (int64_t)c * kChunk;
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int vi = p * NT + tid, row = min(vi / KQV, last), cv = vi % KQV;
            rk[p] = *reinterpret_cast<const V *>(kg + (base + row) * sqk + cv * TR::kVec);
            if (gg) { // the query of the real token, on its last substep only
                const Substep st = substep_at(sb, (uint32_t)(base + row));
                rq[p] = *reinterpret_cast<const V *>(qh + st.t * sqk + cv * TR::kVec);
                qon[p] = st.j == (int)sb.nh - 1;
            } else {
                rq[p] = *reinterpret_cast<const V *>(qg + (base + row) * sqk + cv * TR::kVec);
            }
        }
        if (has_v) {
#pragma unroll
            for (int p = 0; p < NVV; ++p) {
                const int vi = p * NT + tid, row = min(vi / VV, last), cv = vi % VV;
                rv[p] = *reinterpret_cast<const V *>(vg + (base + row) * sv + cv * TR::kVec);
            }
        }
        rbeta = bg[(base + min(tid & (kChunk - 1), last)) * H]; // every wave holds all 64
        if (gg) { // the decay of the real token, on its first substep only
            const Substep st = substep_at(sb, (uint32_t)(base + min(tid & (kChunk - 1), last)));
            rg = gh[st.t * H];
            gon = st.j == 0;
        }
    }
    // Returns lane l's decay prefix sum (gated), else 0.
    __device__ inline float store_kqb(E *Ks, E *Qs, float *Bs, float *Gs) const {
        const V zero = {};
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int vi = p * NT + tid, row = vi / KQV, cv = vi % KQV;
            const bool ok = row < nval;
            *reinterpret_cast<V *>(Ks + row * L::K + cv * TR::kVec) = ok ? rk[p] : zero;
            if (Qs) *reinterpret_cast<V *>(Qs + row * L::K + cv * TR::kVec) = ok && (!gg || qon[p]) ? rq[p] : zero;
        }
        // the four waves write identical values: no branch needed
        const int l = tid & (kChunk - 1);
        Bs[l] = l < nval ? TR::tof(rbeta) : 0.f;
        float gl = 0.f;
        if (gg) {
            // inclusive prefix sum over the chunk's tokens (lane l = token l), in
            // base-2 units; tokens past the end add nothing
            gl = wave_inclusive_sum(l < nval && gon ? rg * 1.44269504088896340736f : 0.f, l);
            if (Gs) Gs[l] = gl;
        }
        return gl;
    }
    __device__ inline void store_q(E *Qs) const {
        const V zero = {};
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int vi = p * NT + tid, row = vi / KQV, cv = vi % KQV;
            *reinterpret_cast<V *>(Qs + row * L::K + cv * TR::kVec) = row < nval && (!gg || qon[p]) ? rq[p] : zero;
        }
    }
    __device__ inline void store_v(E *Vs) const {
        if (!has_v) return;
        const V zero = {};
#pragma unroll
        for (int p = 0; p < NVV; ++p) {
            const int vi = p * NT + tid, row = vi / VV, cv = vi % VV;
            *reinterpret_cast<V *>(Vs + row * L::V + cv * TR::kVec) = row < nval ? rv[p] : zero;
        }
    }
};

template <typename E, int DK, int DV, bool WRITE_O, int NT = kThreads>
__device__ inline Stager<E, DK, NT> make_stager(const ChainArgs &a, const Work &wk, int tid) {
    Stager<E, DK, NT> sg;
    sg.sqk = (int64_t)a.H * DK;
    sg.sv = (int64_t)a.H * DV;
    sg.kg = reinterpret_cast<const E *>(a.k) + wk.tok0 * sg.sqk + (int64_t)wk.h * DK;
    sg.qg = reinterpret_cast<const E *>(a.q) + wk.tok0 * sg.sqk + (int64_t)wk.h * DK;
    sg.vg = reinterpret_cast<const E *>(a.v) + wk.tok0 * sg.sv + (int64_t)wk.h * DV + wk.row0;
    sg.bg = reinterpret_cast<const E *>(a.beta) + wk.tok0 * a.H + wk.h;
    sg.gg = a.g ? a.g + wk.tok0 * a.H + wk.h : nullptr;
    sg.qh = reinterpret_cast<const E *>(a.q) + (int64_t)wk.h * DK;
    sg.gh = a.g ? a.g + wk.h : nullptr;
    sg.sb = a.g ? substep_base(wk.tok0, a.nh) : SubstepBase{0, 0u, 1u};
    sg.rg = 0.f;
    sg.H = a.H;
    sg.len = wk.len;
    sg.tid = tid;
    sg.has_v = WRITE_O || wk.has_v; // outputs are only written by tiles that have V
    sg.rbeta = Tr<E>::fromf(0.f);
    sg.nval = 0;
    return sg;
}

// Sacc[m][i] = S[row0 + 16w + c16][16m + 4g + i]
template <int DK>
__device__ inline void state_in(f32x4 (&Sacc)[DK / 16], const Work &wk, int w, int g, int c16) {
    const int srow = wk.row0 + 16 * w + c16;
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
        if (wk.Sin) {
            Sacc[m] = *reinterpret_cast<const f32x4 *>(wk.Sin + (16 * w + c16) * DK + 16 * m + 4 * g);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[m][i] = (wk.identity && (16 * m + 4 * g + i) == srow) ? 1.f : 0.f;
        }
    }
}
template <int DK>
__device__ inline void state_out(const f32x4 (&Sacc)[DK / 16], const Work &wk, int w, int g, int c16) {
    if (!wk.Sout) return;
    if (!wk.transposed_out) {
#pragma unroll
        for (int m = 0; m < DK / 16; ++m)
            *reinterpret_cast<f32x4 *>(wk.Sout + (16 * w + c16) * DK + 16 * m + 4 * g) = Sacc[m];
    } else {
        const int srow = wk.row0 + 16 * w + c16;
#pragma unroll
        for (int m = 0; m < DK / 16; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) wk.Sout[(int64_t)(16 * m + 4 * g + i) * DK + srow] = Sacc[m][i];
    }
}

// O store: Oacc[t][e] = O[16t + c16][16w + 4g + e] of chunk c. Gated path:
// og is the output at real token 0 and virtual row 64 c + tok of the work is
// stored at its real token on the last substep only.
template <typename E, bool GATED>
__device__ inline void store_o(E *og, int64_t sv, int c, int nval, const SubstepBase &sb, const f32x4 (&Oacc)[4],
                               int w, int g, int c16) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int tok = 16 * t + c16;
        if constexpr (GATED) {
            const Substep st = substep_at(sb, (uint32_t)(c * kChunk + tok));
            if (tok < nval && st.j == (int)sb.nh - 1) stf(og + st.t * sv + 16 * w + 4 * g, Tr<E>::cvt(Oacc[t]));
        } else {
            if (tok < nval) stf(og + ((int64_t)c * kChunk + tok) * sv + 16 * w + 4 * g, Tr<E>::cvt(Oacc[t]));
        }
    }
}

// ---------------------------------------------------------------------------
// Serial kernel: A, B, C, D, E one after the other, one staging buffer.
// ---------------------------------------------------------------------------
template <typename E, int DK> struct SmemSerial {
    using L = Ld<E, DK>;
    static constexpr size_t oKs = 0;
    static constexpr size_t oQs = oKs + L::szK;
    static constexpr size_t oVs = oQs + L::szK;
    static constexpr size_t oBs = oVs + L::szV;
    static constexpr size_t oGs = oBs + sizeof(float) * kChunk; // decay prefix sums
    static constexpr size_t oTs = oGs + sizeof(float) * kChunk;
    static constexpr size_t oPs = oTs + L::szT;
    static constexpr size_t oNs = oPs + L::szT;
    static constexpr size_t oWA = oNs + L::szN;
    static constexpr size_t total = oWA + L::szWA;
};

template <typename E, int DK, int DV, bool WRITE_O, bool GATED>
__global__ __launch_bounds__(kThreads) void chain_kernel_serial(const ChainArgs a) {
    using TR = Tr<E>;
    using F = typename TR::F;
    using PH = Phases<E, DK>;
    using SM = SmemSerial<E, DK>;
    using L = Ld<E, DK>;
    constexpr int NMT = DK / 16;
    static_assert(SM::total <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[SM::total];
    E *Ks = reinterpret_cast<E *>(smem + SM::oKs);
    E *Qs = reinterpret_cast<E *>(smem + SM::oQs);
    E *Vs = reinterpret_cast<E *>(smem + SM::oVs);
    float *Bs = reinterpret_cast<float *>(smem + SM::oBs);
    float *Gs = reinterpret_cast<float *>(smem + SM::oGs);
    E *TsT = reinterpret_cast<E *>(smem + SM::oTs);
    E *Ps = reinterpret_cast<E *>(smem + SM::oPs);
    E *NsT = reinterpret_cast<E *>(smem + SM::oNs);
    float *As = reinterpret_cast<float *>(smem + SM::oWA);
    E *Ws = reinterpret_cast<E *>(smem + SM::oWA);

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const Work wk = decode_work<DK, DV>(a);
    f32x4 Sacc[NMT];
    state_in<DK>(Sacc, wk, w, g, c16);
    const int NC = (wk.len + kChunk - 1) / kChunk;
    auto sg = make_stager<E, DK, DV, WRITE_O>(a, wk, tid);
    const bool has_v = WRITE_O || wk.has_v;
    const int64_t sv = (int64_t)a.H * DV;
    E *og = WRITE_O ? reinterpret_cast<E *>(a.o) + (GATED ? 0 : wk.tok0 * sv) + (int64_t)wk.h * DV + wk.row0
                    : nullptr;

    // T and P are lower triangular and only their lower blocks are written:
    // zero both once so the blocks above the diagonal stay zero.
    for (int i = tid; i < kChunk * L::T; i += kThreads) {
        TsT[i] = TR::fromf(0.f);
        Ps[i] = TR::fromf(0.f);
    }
    if (NC > 0) {
        sg.load(0);
        sg.store_kqb(Ks, Qs, Bs, Gs);
        sg.store_v(Vs);
    }
    __syncthreads();

    f32x4 Zacc[4], Oacc[4];
    for (int c = 0; c < NC; ++c) {
        const int nval = min(kChunk, wk.len - c * kChunk);
        sg.load(min(c + 1, NC - 1)); // next chunk (the last iteration re-reads its own)
        // A
        switch (w) {
#define DN_A(W)                                                                                                \
    case W: {                                                                                                  \
        typename PH::template GramFrags<W> f;                                                                  \
        PH::template gram_fetch<W>(f, Ks, Qs, g, c16);                                                         \
        sched_fence();                                                                                         \
        if (WRITE_O || !(W & 1)) PH::template gram_compute<W, GATED>(f, Bs, Gs, As, Ps, g, c16);               \
    } break;
            DN_A(0) DN_A(1) DN_A(2) DN_A(3)
#undef DN_A
        }
        __syncthreads();
        // B
        F nfrag;
        {
            typename PH::DiagFrags df;
            PH::diag_fetch(df, As, Bs, w, c16);
            sched_fence();
            nfrag = PH::diag_compute(df, NsT, TsT, w, g, c16);
        }
        __syncthreads();
        // C
        switch (w) {
#define DN_C(B)                                                                                                \
    case B: {                                                                                                  \
        typename PH::template OffFrags<B> f;                                                                   \
        PH::template off_fetch<B>(f, As, NsT, Bs, g, c16);                                                     \
        sched_fence();                                                                                         \
        PH::template off_compute<B>(f, nfrag, TsT, g, c16);                                                    \
    } break;
            DN_C(0) DN_C(1) DN_C(2)
#undef DN_C
        default: break;
        }
        __syncthreads();
        // D
        {
            typename PH::WUFrags f;
            PH::template wu_fetch<GATED>(f, Ks, Vs, TsT, Gs, has_v, w, g, c16);
            sched_fence();
            PH::wu_compute(f, Ws, has_v, Zacc, w, g, c16);
        }
        __syncthreads();
        // E
        F SB[NMT], ZB[4];
#pragma unroll
        for (int m = 0; m < NMT; ++m) SB[m] = TR::cvt(Sacc[m]);
        {
            typename PH::ZFrags f;
            PH::z_fetch(f, Ws, g, c16);
            sched_fence();
            PH::z_compute(f, SB, Zacc, ZB);
        }
        if constexpr (WRITE_O) {
            typename PH::OFrags f;
            PH::template o_fetch<GATED>(f, Qs, Ps, Gs, g, c16);
            sched_fence();
            PH::template o_compute<GATED>(f, SB, ZB, Oacc);
            store_o<E, GATED>(og, sv, c, nval, sg.sb, Oacc, w, g, c16);
        }
        {
            typename PH::SFrags f;
            PH::template s_fetch<GATED>(f, Ks, Gs, g, c16);
            sched_fence();
            PH::template s_compute<GATED>(f, ZB, Sacc);
        }
        __syncthreads();
        sg.store_kqb(Ks, Qs, Bs, Gs);
        sg.store_v(Vs);
        __syncthreads();
    }
    state_out<DK>(Sacc, wk, w, g, c16);
}

// Prefix composition of the group maps for one (b, h) and 16 state rows:
//   S_{g+1} = S_g P_g + Q_g,  g = f..G-2,  S_0 = S0 (or zero),
// with f = cp_first (S_f read from ws_S when f > 0: the end state of a group
// that ran its chain ahead of the transitions); writes S_{f+1}..S_{G-1} to ws_S. fp32 throughout (fp32 matrix cores). Wave w
// of DK/16 computes output column tile w, with the contraction split over two
// accumulators (even and odd 16-blocks) so that the dependent product chain
// is half as long; the 16 rows of S are exchanged through LDS between steps.
// The operands of steps g + 1 and g + 2 (P and Q do not depend on the chain)
// are in flight while step g computes.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void compose_kernel(const ChainArgs a) {
    constexpr int LDS_ = DK + 4;
    constexpr int NK = DK / 16, NT = 64 * (DK / 16);
    __shared__ __attribute__((aligned(16))) float Sl[16 * LDS_];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int rb = blockIdx.x % (DV / 16);
    const int bh = blockIdx.x / (DV / 16);
    const int f = a.cp_first;
    const float *Sf = f > 0  ? a.ws_S + ((int64_t)bh * a.G + f) * DV * DK
                      : a.S0 ? a.S0 + (int64_t)bh * DV * DK
                             : nullptr;
    for (int idx = tid; idx < 16 * DK; idx += NT) {
        const int r = idx / DK, col = idx - r * DK;
        Sl[r * LDS_ + col] = Sf ? Sf[(16 * rb + r) * DK + col] : 0.f;
    }
    // p[kk] = P_g^T[16 w + c16][16 kk + 4 g ..], q = Q_g[16 rb + c16][16 w + 4 g ..]; three
    // register sets, step g in set g % 3, so the loads of step g + 2 go into the
    // set step g - 1 has finished with
    f32x4 P0[NK], P1[NK], P2[NK], Q0, Q1, Q2;
    auto load = [&](int gi, f32x4 (&p)[NK], f32x4 &q) {
        const int64_t slot = (int64_t)bh * a.G + gi;
        const float *Pt = a.ws_P + slot * DK * DK;
        const float *Qg = a.ws_Q + (slot * DV + 16 * rb) * DK;
        q = *reinterpret_cast<const f32x4 *>(Qg + c16 * DK + 16 * w + 4 * g);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
            p[kk] = *reinterpret_cast<const f32x4 *>(Pt + (16 * w + c16) * DK + 16 * kk + 4 * g);
    };
    auto step = [&](int gi, const f32x4 (&pc)[NK], const f32x4 &qc, f32x4 (&pl)[NK], f32x4 &ql) {
        f32x4 acc0 = qc, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; kk += 2) {
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(Sl + c16 * LDS_ + 16 * kk + 4 * g);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(Sl + c16 * LDS_ + 16 * kk + 16 + 4 * g);
            acc0 = Tr<float>::mma16(acc0, pc[kk], s0);
            acc1 = Tr<float>::mma16(acc1, pc[kk + 1], s1);
        }
        const f32x4 acc = acc0 + acc1;
        // issued after this step's products, so that waiting for this step's
        // operands never waits for them
        if (gi + 2 < a.G - 1) load(gi + 2, pl, ql);
        // acc[i] = S_{g+1}[row 16 rb + c16][16 w + 4 g + i]
        __syncthreads();
        const int64_t slot = (int64_t)bh * a.G + gi;
        float *Sn = a.ws_S + ((slot + 1) * DV + 16 * rb) * DK;
        *reinterpret_cast<f32x4 *>(Sl + c16 * LDS_ + 16 * w + 4 * g) = acc;
        *reinterpret_cast<f32x4 *>(Sn + c16 * DK + 16 * w + 4 * g) = acc;
        __syncthreads();
    };
    if (a.G > f + 1) load(f, P0, Q0);
    if (a.G > f + 2) load(f + 1, P1, Q1);
    __syncthreads();
    for (int gi = f; gi + 1 < a.G; gi += 3) {
        step(gi, P0, Q0, P2, Q2);
        if (gi + 2 < a.G) step(gi + 1, P1, Q1, P0, Q0);
        if (gi + 3 < a.G) step(gi + 2, P2, Q2, P1, Q1);
    }
}

// Composition of the backward pass's group maps (context-parallel reverse
// chain) for one (b, h) and 16 gradient rows. Over a group the reverse chain
// is affine in the gradient at the group's end, dS_start = dS_end P_g^T + C_g,
// with P_g the group's forward transition (the gradient of S P_g + Q_g with
// respect to S) and C_g the reverse chain's result from a zero end gradient.
//   E_{G-1} = dS_final (or zero),  E_{g-1} = E_g P_g^T + C_g,  g = G-1..1,
// into ws_E (E_g: the gradient at the end of group g). ws_P holds P_g^T, so
// E_g P_g^T is the product with the stored matrix itself: operand A of the
// product reads it down its columns. Layout of the waves as in compose_kernel.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void compose_bwd_kernel(const BwdArgs a) {
    constexpr int LDS_ = DK + 4;
    constexpr int NK = DK / 16, NT = 64 * (DK / 16);
    __shared__ __attribute__((aligned(16))) float El[16 * LDS_];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int rb = blockIdx.x % (DV / 16);
    const int bh = blockIdx.x / (DV / 16);
    for (int idx = tid; idx < 16 * DK; idx += NT) {
        const int r = idx / DK, col = idx - r * DK;
        El[r * LDS_ + col] = a.dS_final ? a.dS_final[((int64_t)bh * DV + 16 * rb + r) * DK + col] : 0.f;
    }
    // p[kk][j] = (P_g^T)[16 kk + 4 g + j][16 w + c16], c = C_g[16 rb + c16][16 w + 4 g ..]
    f32x4 pa[NK], ca, pn[NK], cn;
    auto load = [&](int gi, f32x4 (&p)[NK], f32x4 &c) {
        const int64_t slot = (int64_t)bh * a.G + gi;
        const float *W = a.ws_P + slot * DK * DK;
        c = *reinterpret_cast<const f32x4 *>(a.ws_C + (slot * DV + 16 * rb + c16) * DK + 16 * w + 4 * g);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) p[kk][j] = W[(16 * kk + 4 * g + j) * DK + 16 * w + c16];
    };
    if (a.G > 1) load(a.G - 1, pn, cn);
    __syncthreads();
    for (int gi = a.G - 1; gi >= 1; --gi) {
        ca = cn;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) pa[kk] = pn[kk];
        f32x4 acc0 = ca, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; kk += 2) {
            const f32x4 e0 = *reinterpret_cast<const f32x4 *>(El + c16 * LDS_ + 16 * kk + 4 * g);
            const f32x4 e1 = *reinterpret_cast<const f32x4 *>(El + c16 * LDS_ + 16 * kk + 16 + 4 * g);
            acc0 = Tr<float>::mma16(acc0, pa[kk], e0);
            acc1 = Tr<float>::mma16(acc1, pa[kk + 1], e1);
        }
        const f32x4 acc = acc0 + acc1; // acc[i] = E_{g-1}[16 rb + c16][16 w + 4 g + i]
        if (gi >= 2) load(gi - 1, pn, cn);
        __syncthreads();
        float *En = a.ws_E + (((int64_t)bh * a.G + gi - 1) * DV + 16 * rb) * DK;
        *reinterpret_cast<f32x4 *>(El + c16 * LDS_ + 16 * w + 4 * g) = acc;
        *reinterpret_cast<f32x4 *>(En + c16 * DK + 16 * w + 4 * g) = acc;
        __syncthreads();
    }
}

template <int DK, int DV, bool WO> hipError_t launch_one(const ChainArgs &a, hipStream_t s) {
    const int grid = a.n_units * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    if (a.g)
        hipLaunchKernelGGL((chain_kernel_serial<float, DK, DV, WO, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((chain_kernel_serial<float, DK, DV, WO, false>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <bool WO> hipError_t launch_dims_f32(int dk, int dv, const ChainArgs &a, hipStream_t s) {
    if (dk == 64 && dv == 128) return launch_one<64, 128, WO>(a, s);
    if (dk == 64 && dv == 64) return launch_one<64, 64, WO>(a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Backward pass (bf16 operands, fp32 accumulation).
//
// The pages give no backward pass; these kernels apply the chain rule to the
// per-chunk algorithm of "Linear Attention, Visualized", DeltaNet > "Complete
// per-chunk algorithm", in the form the forward kernels use (state S,
// dv x dk; P = (Q K^T) lower-inclusive; T = (I + A)^-1 diag(beta) with
// A = diag(beta) (K K^T) strictly lower):
//   Y = V - K S^T,  Z = T Y,  O = Q S^T + P Z,  S' = S + Z^T K.
// For upstream dO (chunk) and dS' (state after the chunk):
//   dZ = P^T dO + K dS'^T,  dY = T^T dZ,  dV = dY,
//   dS = dS' + dO^T Q - dY^T K                        (the reverse chain)
//   dP = dO Z^T (lower-inclusive),  dT = dZ Y^T (lower-inclusive),
//   dQ = dO S + dP K,  dK = dP^T Q + Z dS' - dY S + (dL + dL^T) K,
// and through T = N diag(beta), N = (I + A)^-1, A = diag(beta) L:
//   X = N^T dT,  dbeta_i = X_ii + sum_j dA_ij L_ij,  dA = -(X diag(beta)) N^T
//   (strictly lower),  dL = diag(beta) dA.
// Pass 1 is the forward chain kernel without output, keeping the state that
// enters every chunk and the chunk's T^T (as the forward formed it). Pass 2
// (bwd_chain_kernel) walks the chunks backwards per (unit, 64 value rows),
// carrying dS in registers; it takes T^T from pass 1, forms P, and writes dV
// and, per chunk, the sums over its 64 value rows of dP, dT, dO S and
// Z dS' - dY S. Pass 3 (bwd_finish_kernel, one workgroup per chunk) adds those
// partial sums over the value tiles, forms N^T = I - L^T T^T (from
// N (I + diag(beta) L) = I, so no triangular solve) and finishes dQ, dK and
// dbeta.
// ---------------------------------------------------------------------------
__device__ inline f32x4 widen_bf16(bf16x4 x) { return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }

template <int DK, bool GATED> struct BwdLds {
    using L = Ld<__bf16, DK>;
    static constexpr int LT = L::T; // stride of the 64-wide bf16 tiles
    static constexpr size_t oK = 0, oQ = oK + L::szK, oV = oQ + L::szK, oD = oV + L::szV, oB = oD + L::szV;
    static constexpr size_t oT = oB + 256, oP = oT + L::szT;
    static constexpr size_t oX = oP + L::szT; // Y, Z, dZ, dY tiles
    static constexpr size_t oS = oX + 4 * L::szT, oR = oS + L::szK;
    // gated: decay prefix sums (the row-scaled dO tile replaces V once Y is formed)
    static constexpr size_t oG = oR + L::szK;
    static constexpr size_t total = GATED ? oG + 256 : oR + L::szK;
};

// A bf16 vector with every element times f.
__device__ inline bf16x8 scale8(bf16x8 x, float f) {
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (__bf16)((float)x[e] * f);
    return y;
}

// SUB: several substeps per real token (Gated Delta Product), so queries,
// decays and output gradients are addressed through the substep map.
template <int DK, int DV, bool GATED, bool SUB>
__global__ __launch_bounds__(kThreads) void bwd_chain_kernel(const BwdArgs a) {
    using E = __bf16;
    using TR = Tr<E>;
    using F = typename TR::F;
    using L = Ld<E, DK>;
    using LY = BwdLds<DK, GATED>;
    constexpr int NMT = DK / 16, LT = LY::LT;
    static_assert(LY::total <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::total];
    E *Ks = reinterpret_cast<E *>(smem + LY::oK), *Qs = reinterpret_cast<E *>(smem + LY::oQ);
    E *Vs = reinterpret_cast<E *>(smem + LY::oV), *Ds = reinterpret_cast<E *>(smem + LY::oD);
    float *Bs = reinterpret_cast<float *>(smem + LY::oB);
    E *TsT = reinterpret_cast<E *>(smem + LY::oT), *Ps = reinterpret_cast<E *>(smem + LY::oP);
    E *Ys = reinterpret_cast<E *>(smem + LY::oX), *Zs = Ys + 64 * LT, *dZs = Zs + 64 * LT, *dYs = dZs + 64 * LT;
    E *Ss = reinterpret_cast<E *>(smem + LY::oS), *Rs = reinterpret_cast<E *>(smem + LY::oR);
    // gated: prefix sums gamma (base 2), and diag(exp(gamma)) dO over V after Y;
    // ungated: dO itself
    float *Gs = GATED ? reinterpret_cast<float *>(smem + LY::oG) : nullptr;
    E *Dgs = GATED ? Vs : Ds;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    int u, tau;
    // units: (sequence, head), or (b, h, group) for the context-parallel kinds
    // (groups 1..G-1 for kRevCpAffine, all G for kRevCpRun)
    const int cp_groups = a.rev_kind == kRevChain ? 1 : (a.rev_kind == kRevCpAffine ? a.G - 1 : a.G);
    map_block(blockIdx.x, a.B * a.H * cp_groups, a.n_tiles, u, tau); // the tiles of a unit share an XCD
    const int row0 = 64 * tau;
    // token range, state slot su and first chunk slot of this unit; the
    // gradient at the end of the range (gin, nullptr: zero), where the one at
    // its start goes (gout), and whether dv and the partial sums are written
    int rank, h;
    int64_t tok0, su, slot0;
    int len;
    const float *gin;
    float *gout;
    bool store = true;
    if (a.rev_kind != kRevChain) {
        const int bh = u / cp_groups;
        const int gi = u - bh * cp_groups + (a.rev_kind == kRevCpAffine ? 1 : 0);
        rank = bh / a.H;
        h = bh - rank * a.H;
        const int t_begin = gi * a.cpg * kChunk;
        tok0 = (int64_t)rank * a.T + t_begin;
        len = min(a.T, (gi + 1) * a.cpg * kChunk) - t_begin;
        su = bh;
        slot0 = (int64_t)bh * a.NC + (int64_t)gi * a.cpg;
        if (a.rev_kind == kRevCpAffine) {
            gin = nullptr;
            gout = a.ws_C + (((int64_t)bh * a.G + gi) * DV + row0) * DK;
            store = false;
        } else {
            gin = gi == a.G - 1 ? (a.dS_final ? a.dS_final + ((int64_t)bh * DV + row0) * DK : nullptr)
                                : a.ws_E + (((int64_t)bh * a.G + gi) * DV + row0) * DK;
            gout = gi == 0 && a.dS0 ? a.dS0 + ((int64_t)bh * DV + row0) * DK : nullptr;
        }
    } else {
        rank = u / a.H;
        h = u - rank * a.H;
        if (a.cu_seqlens) {
            const int n = a.seq_order ? a.seq_order[rank] : rank;
            tok0 = a.cu_seqlens[n];
            len = a.cu_seqlens[n + 1] - a.cu_seqlens[n];
            su = (int64_t)n * a.H + h;
            slot0 = (int64_t)a.chunk_base[n] * a.H + (int64_t)h * ((len + kChunk - 1) / kChunk);
        } else {
            tok0 = (int64_t)rank * a.T;
            len = a.T;
            su = u;
            slot0 = (int64_t)u * a.NC;
        }
        gin = a.dS_final ? a.dS_final + (su * DV + row0) * DK : nullptr;
        gout = a.dS0 ? a.dS0 + (su * DV + row0) * DK : nullptr;
    }
    const int NC = (len + kChunk - 1) / kChunk;
    const int64_t sqk = (int64_t)a.H * DK, sv = (int64_t)a.H * DV;

    Stager<E, DK> sg;
    sg.sqk = sqk;
    sg.sv = sv;
    sg.kg = reinterpret_cast<const E *>(a.k) + tok0 * sqk + (int64_t)h * DK;
    sg.qg = reinterpret_cast<const E *>(a.q) + tok0 * sqk + (int64_t)h * DK;
    sg.vg = reinterpret_cast<const E *>(a.v) + tok0 * sv + (int64_t)h * DV + row0;
    sg.bg = reinterpret_cast<const E *>(a.beta) + tok0 * a.H + h;
    sg.gg = nullptr;
    sg.qh = nullptr;
    sg.gh = nullptr;
    sg.sb = SubstepBase{0, 0u, 1u};
    sg.H = a.H;
    sg.len = len;
    sg.tid = tid;
    sg.has_v = true;
    sg.rbeta = TR::fromf(0.f);
    sg.rg = 0.f;
    sg.nval = 0;
    if constexpr (GATED) { // decays (and so queries) addressed by real token
        sg.gg = a.g;
        sg.gh = a.g + h;
        sg.qh = reinterpret_cast<const E *>(a.q) + (int64_t)h * DK;
        sg.sb = SUB ? substep_base(tok0, a.nh) : SubstepBase{tok0, 0u, 1u};
    }
    const E *dOg = reinterpret_cast<const E *>(a.dO) + tok0 * sv + (int64_t)h * DV + row0;
    const E *dOh = reinterpret_cast<const E *>(a.dO) + (int64_t)h * DV + row0; // real token 0 (substeps)
    E *dVg = reinterpret_cast<E *>(a.dv) + tok0 * sv + (int64_t)h * DV + row0;

    // dS rows 16w + c16 of this tile: dSacc[m][i] = dS[row0 + 16w + c16][16m + 4g + i]
    // Sraw: the bf16 state entering the chunk, kept as loaded (the load is not
    // waited for until the chunk's first use of it)
    f32x4 dSacc[NMT];
    bf16x4 Sraw[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
        dSacc[m] = gin ? *reinterpret_cast<const f32x4 *>(gin + (16 * w + c16) * DK + 16 * m + 4 * g)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = tid; i < kChunk * LT; i += kThreads) Ps[i] = TR::fromf(0.f); // only P's lower blocks are written

    // HBM loads of chunk c (K, Q, V, beta, dO and the state entering it) into
    // registers; issued one chunk ahead so their latency hides under the
    // previous chunk's products.
    typename TR::V dov[2], tv[2];
    bool don[2] = {true, true}; // substeps: the row is its real token's last substep (applied at staging)
    const E *Tg = a.T_chunks + slot0 * kChunk * kChunk;
    auto load_chunk = [&](int c) {
        const int n = min(kChunk, len - c * kChunk);
        sg.load(c);
#pragma unroll
        for (int p = 0; p < 2; ++p) // T^T of the chunk, as the forward pass formed it
            tv[p] = *reinterpret_cast<const typename TR::V *>(Tg + (int64_t)c * kChunk * kChunk + 8 * (p * kThreads + tid));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int vi = p * kThreads + tid, row = vi / 8, cv = vi % 8;
            const int64_t x = (int64_t)c * kChunk + min(row, n - 1);
            if constexpr (SUB) { // the output gradient of the real token, on its last substep only
                const Substep st = substep_at(sg.sb, (uint32_t)x);
                dov[p] = *reinterpret_cast<const typename TR::V *>(dOh + st.t * sv + 8 * cv);
                don[p] = st.j == a.nh - 1;
            } else {
                dov[p] = *reinterpret_cast<const typename TR::V *>(dOg + x * sv + 8 * cv);
            }
        }
        const E *Sr = a.S_chunks16 + ((slot0 + c) * DV + row0 + 16 * w + c16) * DK + 4 * g;
#pragma unroll
        for (int m = 0; m < NMT; ++m) Sraw[m] = *reinterpret_cast<const bf16x4 *>(Sr + 16 * m);
    };
    if (NC > 0) load_chunk(NC - 1);
    for (int r = NC - 1; r >= 0; --r) {
        const int nval = min(kChunk, len - r * kChunk);
        __syncthreads(); // the previous chunk's reads of the staging buffers are done
        const float gl = sg.store_kqb(Ks, Qs, Bs, Gs); // gated: gamma of token `lane`
        sg.store_v(Vs);
        // gated: gamma_C (the chunk's last prefix sum; tokens past the end add nothing)
        const float gC = GATED ? __shfl(gl, 63) : 0.f, eC = GATED ? __builtin_amdgcn_exp2f(gC) : 1.f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int vi = p * kThreads + tid, row = vi / 8, cv = vi % 8;
            *reinterpret_cast<typename TR::V *>(Ds + row * L::V + 8 * cv) =
                row < nval && (!SUB || don[p]) ? dov[p] : typename TR::V{};
            *reinterpret_cast<typename TR::V *>(TsT + row * L::T + 8 * cv) = tv[p];
        }
        // This wave's 16 value rows (column c16 of the accumulators).
        F SBn[NMT], dSB[NMT], YB[4], dZB[4], dYBn[4];
        f32x4 acc[4];
        float sdot = 0.f; // gated: this lane's share of <dS', S>
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            const f32x4 Sm = widen_bf16(Sraw[m]);
            stf(Ss + (16 * w + c16) * L::K + 16 * m + 4 * g, Sraw[m]);
            stf(Rs + (16 * w + c16) * L::K + 16 * m + 4 * g, TR::cvt(dSacc[m])); // dS after the chunk
            SBn[m] = -Sraw[m];
            dSB[m] = TR::cvt(dSacc[m]);
            if constexpr (GATED)
#pragma unroll
                for (int i = 0; i < 4; ++i) sdot += dSacc[m][i] * Sm[i];
        }
        __syncthreads();
        if (r > 0) load_chunk(r - 1);
        // the masked scores P = (Q K^T) lower-inclusive (T^T came with the
        // chunk): the ten 16x16 tiles (a, c <= a), three or two per wave
        {
            constexpr int NKB = DK / 32;
            const int nt = w < 2 ? 3 : 2;
#pragma unroll
            for (int it = 0; it < 3; ++it) {
                if (it >= nt) break;
                // wave 0: (0,0) (3,0) (3,1); 1: (1,0) (1,1) (3,2); 2: (2,0) (2,1); 3: (2,2) (3,3)
                const int code = w == 0 ? (it == 0 ? 0x00 : it == 1 ? 0x30 : 0x31)
                               : w == 1 ? (it == 0 ? 0x10 : it == 1 ? 0x11 : 0x32)
                               : w == 2 ? (it == 0 ? 0x20 : 0x21)
                                        : (it == 0 ? 0x22 : 0x33);
                const int ab = code >> 4, cb = code & 15;
                F kf[NKB][2], qf[NKB][2];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        kf[kb][h2] = ldrow(Ks, L::K, 16 * cb + c16, 32 * kb + 16 * h2, g);
                        qf[kb][h2] = ldrow(Qs, L::K, 16 * ab + c16, 32 * kb + 16 * h2, g);
                    }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) acc = TR::mma32(acc, kf[kb][0], kf[kb][1], qf[kb][0], qf[kb][1]);
                // acc[e] = k_{16cb + 4g + e} . q_{16ab + c16}
                const int row = 16 * ab + c16, col = 16 * cb + 4 * g;
                if constexpr (GATED) { // times exp(gamma_row - gamma_col)
                    const float gr = Gs[row];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[e] = (col + e > row) ? 0.f : acc[e] * __builtin_amdgcn_exp2f(gr - Gs[col + e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = (col + e > row) ? 0.f : acc[e];
                }
                stf(Ps + row * L::T + col, TR::cvt(acc));
            }
        }
        __syncthreads();
        // Y = V - K S^T (gated: V - diag(exp(gamma)) K S^T). eg[t][i] = exp(gamma)
        // and ez[t][i] = exp(gamma_C - gamma) of token 16t + 4g + i (gated).
        f32x4 eg[4], ez[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (GATED) {
                const f32x4 gq = *reinterpret_cast<const f32x4 *>(Gs + 16 * t + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    eg[t][i] = __builtin_amdgcn_exp2f(gq[i]);
                    ez[t][i] = __builtin_amdgcn_exp2f(gC - gq[i]);
                }
            }
            acc[t] = GATED ? f32x4{0.f, 0.f, 0.f, 0.f} : widen_bf16(TR::ldcol(Vs, L::V, 16 * t, 16 * w, g, c16));
#pragma unroll
            for (int kb = 0; kb < NMT / 2; ++kb)
                acc[t] = TR::mma32(acc[t], ldrow(Ks, L::K, 16 * t + c16, 32 * kb, g),
                                   ldrow(Ks, L::K, 16 * t + c16, 32 * kb + 16, g), SBn[2 * kb], SBn[2 * kb + 1]);
            if constexpr (GATED) acc[t] = widen_bf16(TR::ldcol(Vs, L::V, 16 * t, 16 * w, g, c16)) + eg[t] * acc[t];
            YB[t] = TR::cvt(acc[t]);
#pragma unroll
            for (int i = 0; i < 4; ++i) Ys[(16 * t + 4 * g + i) * LT + 16 * w + c16] = YB[t][i];
        }
        if constexpr (GATED) {
            // diag(exp(gamma)) dO into this wave's value columns of V, which only
            // this wave's Y products above read (token `lane`)
            const float f = __builtin_amdgcn_exp2f(gl);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const bf16x8 x = *reinterpret_cast<const bf16x8 *>(Ds + lane * L::V + 16 * w + 8 * h2);
                *reinterpret_cast<bf16x8 *>(Vs + lane * L::V + 16 * w + 8 * h2) = scale8(x, f);
            }
        }
        // Z = T Y
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 <= t; ++s2) z = TR::mma16(z, TR::ldcol(TsT, L::T, 16 * s2, 16 * t, g, c16), YB[s2]);
            const F zb = TR::cvt(z);
#pragma unroll
            for (int i = 0; i < 4; ++i) Zs[(16 * t + 4 * g + i) * LT + 16 * w + c16] = zb[i];
        }
        // dZ = P^T dO + K dS'^T. The two parts use different product shapes and
        // so accumulate separately: a chain that feeds one shape's result to
        // the other as accumulator is not kept apart by the compiler's wait
        // states and gives wrong sums.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 zp = {0.f, 0.f, 0.f, 0.f}, zk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = t; s2 < 4; ++s2)
                zp = TR::mma16(zp, TR::ldcol(Ps, L::T, 16 * s2, 16 * t, g, c16), TR::ldcol(Ds, L::V, 16 * s2, 16 * w, g, c16));
#pragma unroll
            for (int m = 0; m < NMT; m += 2)
                zk = TR::mma32(zk, ldrow(Ks, L::K, 16 * t + c16, 16 * m, g), ldrow(Ks, L::K, 16 * t + c16, 16 * m + 16, g),
                               dSB[m], dSB[m + 1]);
            const f32x4 z = GATED ? zp + ez[t] * zk : zp + zk; // gated: K rows scaled by exp(gamma_C - gamma)
            dZB[t] = TR::cvt(z);
#pragma unroll
            for (int i = 0; i < 4; ++i) dZs[(16 * t + 4 * g + i) * LT + 16 * w + c16] = dZB[t][i];
        }
        // dY = T^T dZ; dV = dY
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = t; s2 < 4; ++s2) z = TR::mma16(z, ldrow(TsT, L::T, 16 * t + c16, 16 * s2, g), dZB[s2]);
            const F yb = TR::cvt(z);
            // gated: the state-side uses of dY take the row factor exp(gamma)
            const f32x4 zs = GATED ? eg[t] * z : z;
            dYBn[t] = TR::cvt(-zs);
            const F ysb = GATED ? TR::cvt(zs) : yb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * t + 4 * g + i;
                dYs[tok * LT + 16 * w + c16] = ysb[i];
                if (store && tok < nval) dVg[((int64_t)r * kChunk + tok) * sv + 16 * w + c16] = yb[i];
            }
        }
        // dS <- dS' + dO^T Q - dY^T K (gated: exp(gamma_C) dS' + (diag(exp(gamma)) dO)^T Q
        // - (diag(exp(gamma)) dY)^T K)
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            if constexpr (GATED) dSacc[m] *= eC;
#pragma unroll
            for (int s2 = 0; s2 < 4; s2 += 2) { // 16x16x32 products over token blocks s2, s2 + 1
                dSacc[m] = TR::mma32(dSacc[m], TR::ldcol(Qs, L::K, 16 * s2, 16 * m, g, c16),
                                     TR::ldcol(Qs, L::K, 16 * s2 + 16, 16 * m, g, c16),
                                     TR::ldcol(Dgs, L::V, 16 * s2, 16 * w, g, c16),
                                     TR::ldcol(Dgs, L::V, 16 * s2 + 16, 16 * w, g, c16));
                dSacc[m] = TR::mma32(dSacc[m], TR::ldcol(Ks, L::K, 16 * s2, 16 * m, g, c16),
                                     TR::ldcol(Ks, L::K, 16 * s2 + 16, 16 * m, g, c16), dYBn[s2], dYBn[s2 + 1]);
            }
        }
        __syncthreads(); // Y, Z, dZ, dY tiles complete

        if (store) { // context-parallel affine runs need only the gradient at the group's start
            // Sums over this tile's 64 value rows, token rows 16w .. 16w + 15 per wave,
            // stored in accumulator order: one 16-byte piece per (wave, column
            // block, lane), so every store (and the finishing kernel's load) of a
            // wave moves 1 KB of contiguous memory.
            E *pb = reinterpret_cast<E *>(a.part + ((int64_t)tau * a.max_slots + slot0 + r) * bwd_part_bytes(DK));
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                if (s2 > w) break; // dP and dT are lower-inclusive: tiles right of the diagonal are zero
                f32x4 dp = {0.f, 0.f, 0.f, 0.f}, dt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kv = 0; kv < 4; kv += 2) { // 16x16x32 products over value blocks kv, kv + 1
                    dp = TR::mma32(dp, ldrow(Ds, L::V, 16 * w + c16, 16 * kv, g), ldrow(Ds, L::V, 16 * w + c16, 16 * kv + 16, g),
                                   ldrow(Zs, LT, 16 * s2 + c16, 16 * kv, g), ldrow(Zs, LT, 16 * s2 + c16, 16 * kv + 16, g));
                    dt = TR::mma32(dt, ldrow(dZs, LT, 16 * w + c16, 16 * kv, g), ldrow(dZs, LT, 16 * w + c16, 16 * kv + 16, g),
                                   ldrow(Ys, LT, 16 * s2 + c16, 16 * kv, g), ldrow(Ys, LT, 16 * s2 + c16, 16 * kv + 16, g));
                }
                *reinterpret_cast<bf16x4 *>(pb + ((w * 4 + s2) * 64 + lane) * 4) = TR::cvt(dp);
                *reinterpret_cast<bf16x4 *>(pb + 4096 + ((w * 4 + s2) * 64 + lane) * 4) = TR::cvt(dt);
            }
            // gated: k . a and k . b per token (a = the Z dS' rows scaled by
            // exp(gamma_C - gamma), b = the dY S rows scaled by exp(gamma))
            f32x4 ska = {0.f, 0.f, 0.f, 0.f}, skb = {0.f, 0.f, 0.f, 0.f};
            f32x4 ezw = {1.f, 1.f, 1.f, 1.f};
            if constexpr (GATED) {
                const f32x4 gq = *reinterpret_cast<const f32x4 *>(Gs + 16 * w + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) ezw[i] = __builtin_amdgcn_exp2f(gC - gq[i]);
            }
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                f32x4 dq = {0.f, 0.f, 0.f, 0.f}, dk1 = {0.f, 0.f, 0.f, 0.f}, dk2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kv = 0; kv < 4; kv += 2) { // 16x16x32 products over value blocks kv, kv + 1
                    const F s0 = TR::ldcol(Ss, L::K, 16 * kv, 16 * m, g, c16), s1 = TR::ldcol(Ss, L::K, 16 * kv + 16, 16 * m, g, c16);
                    dq = TR::mma32(dq, ldrow(Dgs, L::V, 16 * w + c16, 16 * kv, g), ldrow(Dgs, L::V, 16 * w + c16, 16 * kv + 16, g),
                                   s0, s1);
                    dk1 = TR::mma32(dk1, ldrow(Zs, LT, 16 * w + c16, 16 * kv, g), ldrow(Zs, LT, 16 * w + c16, 16 * kv + 16, g),
                                    TR::ldcol(Rs, L::K, 16 * kv, 16 * m, g, c16), TR::ldcol(Rs, L::K, 16 * kv + 16, 16 * m, g, c16));
                    dk2 = TR::mma32(dk2, ldrow(dYs, LT, 16 * w + c16, 16 * kv, g), ldrow(dYs, LT, 16 * w + c16, 16 * kv + 16, g),
                                    s0, s1);
                }
                if constexpr (GATED) {
                    dk1 *= ezw;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float kk = (float)Ks[(16 * w + 4 * g + i) * L::K + 16 * m + c16];
                        ska[i] += kk * dk1[i];
                        skb[i] += kk * dk2[i];
                    }
                }
                *reinterpret_cast<bf16x4 *>(pb + 8192 + ((w * NMT + m) * 64 + lane) * 4) = TR::cvt(dq);
                *reinterpret_cast<bf16x4 *>(pb + 8192 + 64 * DK + ((w * NMT + m) * 64 + lane) * 4) = TR::cvt(dk1 - dk2);
            }
            if constexpr (GATED) {
                float *px = reinterpret_cast<float *>(pb + bwd_part_elems(DK));
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) {
                        ska[i] += __shfl_xor(ska[i], o, 16);
                        skb[i] += __shfl_xor(skb[i], o, 16);
                    }
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) sdot += __shfl_xor(sdot, o, 64);
                if (c16 == 0) {
                    *reinterpret_cast<f32x4 *>(px + 16 * w + 4 * g) = ska;
                    *reinterpret_cast<f32x4 *>(px + 64 + 16 * w + 4 * g) = skb;
                }
                if (lane == 0) px[128 + w] = eC * sdot;
            }
        }
    }
    if (gout) {
#pragma unroll
        for (int m = 0; m < NMT; ++m)
            *reinterpret_cast<f32x4 *>(gout + (16 * w + c16) * DK + 16 * m + 4 * g) = dSacc[m];
    }
}

template <int DK, bool GATED> struct FinLds {
    using L = Ld<__bf16, DK>;
    static constexpr int LT = L::T;
    static constexpr size_t szX = sizeof(__bf16) * 64 * LT;
    // Q is staged only for the last products, over the T and X tiles (adjacent,
    // both dead by then), so that two workgroups fit in a CU's LDS.
    static constexpr size_t oK = 0, oB = oK + L::szK, oBt = oB + 256, oDa = oBt + 256;
    static constexpr size_t oT = oDa + 256, oXs = oT + L::szT;
    static constexpr size_t oP = oXs + szX, oDT = oP + szX, oL = oDT + szX;
    static_assert(L::szT + szX >= L::szK, "Q fits over the T and X tiles");
    // gated: per token (row sum of F) + q . dQ, and per wave the column sums of F
    static constexpr size_t oRq = oL + szX, oCs = oRq + 256;
    static constexpr size_t total = GATED ? oCs + 4 * 256 : oL + szX;
};

template <int DK, int DV, bool GATED, bool SUB>
__global__ __launch_bounds__(kThreads) void bwd_finish_kernel(const BwdArgs a) {
    using E = __bf16;
    using TR = Tr<E>;
    using F = typename TR::F;
    using L = Ld<E, DK>;
    using LY = FinLds<DK, GATED>;
    constexpr int NMT = DK / 16, LT = LY::LT;
    static_assert(LY::total <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::total];
    E *Ks = reinterpret_cast<E *>(smem + LY::oK);
    E *Qs = reinterpret_cast<E *>(smem + LY::oT); // staged late
    float *Bs = reinterpret_cast<float *>(smem + LY::oB), *Bt = reinterpret_cast<float *>(smem + LY::oBt);
    float *dba = reinterpret_cast<float *>(smem + LY::oDa);
    E *TsT = reinterpret_cast<E *>(smem + LY::oT); // N^T once formed
    E *dPs = reinterpret_cast<E *>(smem + LY::oP), *dTs = reinterpret_cast<E *>(smem + LY::oDT);
    E *Xs = reinterpret_cast<E *>(smem + LY::oXs), *dLs = reinterpret_cast<E *>(smem + LY::oL);
    float *Rq = GATED ? reinterpret_cast<float *>(smem + LY::oRq) : nullptr;
    float *Cs = GATED ? reinterpret_cast<float *>(smem + LY::oCs) : nullptr;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    // chunk slot s = blockIdx.x -> sequence, head h and chunk r
    const int64_t s = blockIdx.x;
    int64_t tok0;
    int len, h, r;
    if (a.cu_seqlens) {
        // slots of sequence n: [cb[n] H, cb[n + 1] H), head-major; the grid covers
        // the workspace's slot count, an upper bound, so trailing workgroups idle
        const int32_t *cb = a.chunk_base;
        if (s >= (int64_t)cb[a.B] * a.H) return;
        int lo = 0, hi = a.B - 1; // largest n with cb[n] H <= s
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)cb[mid] * a.H <= s) lo = mid; else hi = mid - 1;
        }
        const int n = lo, ncn = cb[n + 1] - cb[n];
        const int64_t off = s - (int64_t)cb[n] * a.H;
        h = (int)(off / ncn);
        r = (int)(off - (int64_t)h * ncn);
        tok0 = a.cu_seqlens[n];
        len = a.cu_seqlens[n + 1] - a.cu_seqlens[n];
    } else {
        const int u = (int)(s / a.NC), b = u / a.H;
        r = (int)(s - (int64_t)u * a.NC);
        h = u - b * a.H;
        tok0 = (int64_t)b * a.T;
        len = a.T;
    }
    const int64_t sqk = (int64_t)a.H * DK;
    const int nval = min(kChunk, len - r * kChunk);

    Stager<E, DK> sg;
    sg.sqk = sqk;
    sg.sv = 0;
    sg.kg = reinterpret_cast<const E *>(a.k) + tok0 * sqk + (int64_t)h * DK;
    sg.qg = reinterpret_cast<const E *>(a.q) + tok0 * sqk + (int64_t)h * DK;
    sg.vg = nullptr;
    sg.bg = reinterpret_cast<const E *>(a.beta) + tok0 * a.H + h;
    sg.gg = nullptr;
    sg.qh = nullptr;
    sg.gh = nullptr;
    sg.sb = SubstepBase{0, 0u, 1u};
    sg.H = a.H;
    sg.len = len;
    sg.tid = tid;
    sg.has_v = false;
    sg.rbeta = TR::fromf(0.f);
    sg.rg = 0.f;
    sg.nval = 0;
    if constexpr (GATED) { // decays (and so queries) addressed by real token
        sg.gg = a.g;
        sg.gh = a.g + h;
        sg.qh = reinterpret_cast<const E *>(a.q) + (int64_t)h * DK;
        sg.sb = SUB ? substep_base(tok0, a.nh) : SubstepBase{tok0, 0u, 1u};
    }
    sg.load(r);
    typename TR::V tv[2]; // T^T of the chunk, as the forward pass formed it
#pragma unroll
    for (int p = 0; p < 2; ++p)
        tv[p] = *reinterpret_cast<const typename TR::V *>(a.T_chunks + s * kChunk * kChunk +
                                                          8 * (p * kThreads + tid));
    // Partial sums over the value tiles (the chain kernel's accumulator
    // order): dP, dT (lower-inclusive, to LDS) and dQ, dK (this wave's token
    // rows, in registers). Every load is issued before the first use.
    constexpr int NT = DV / 64;
    const E *pbt[NT];
#pragma unroll
    for (int tau = 0; tau < NT; ++tau)
        pbt[tau] = reinterpret_cast<const E *>(a.part + ((int64_t)tau * a.max_slots + s) * bwd_part_bytes(DK));
    auto ld4 = [&](int tau, int off) {
        return widen_bf16(*reinterpret_cast<const bf16x4 *>(pbt[tau] + off + lane * 4));
    };
    f32x4 pp[4], tt[4], dQa[NMT], dKa[NMT];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) { // tiles right of the diagonal are neither stored nor loaded
        pp[s2] = s2 <= w ? ld4(0, (w * 4 + s2) * 256) : f32x4{0.f, 0.f, 0.f, 0.f};
        tt[s2] = s2 <= w ? ld4(0, 4096 + (w * 4 + s2) * 256) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
        dQa[m] = ld4(0, 8192 + (w * NMT + m) * 256);
        dKa[m] = ld4(0, 8192 + 64 * DK + (w * NMT + m) * 256);
    }
#pragma unroll
    for (int tau = 1; tau < NT; ++tau) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            if (s2 <= w) {
                pp[s2] += ld4(tau, (w * 4 + s2) * 256);
                tt[s2] += ld4(tau, 4096 + (w * 4 + s2) * 256);
            }
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            dQa[m] += ld4(tau, 8192 + (w * NMT + m) * 256);
            dKa[m] += ld4(tau, 8192 + 64 * DK + (w * NMT + m) * 256);
        }
    }
    // gated: per token k . a, k . b (summed over the value tiles, wave 0's lanes)
    // and the tiles' exp(gamma_C) <dS', S> shares
    float xa = 0.f, xb = 0.f, xs = 0.f;
    if constexpr (GATED) {
        if (w == 0) {
#pragma unroll
            for (int tau = 0; tau < NT; ++tau) {
                const float *px = reinterpret_cast<const float *>(pbt[tau] + bwd_part_elems(DK));
                xa += px[lane];
                xb += px[64 + lane];
                xs += lane < 4 ? px[128 + lane] : 0.f;
            }
        }
    }
    E *TtS = Xs, *Ls = dLs; // T^T and L until N^T is formed (X and dL come later)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int vi = p * kThreads + tid, row = vi / 8, cv = vi % 8;
        *reinterpret_cast<typename TR::V *>(TtS + row * LT + 8 * cv) = tv[p];
    }
    const float gl = sg.store_kqb(Ks, nullptr, Bs, nullptr); // gated: gamma (base 2) of token `lane`
    // gated: decay factor exp(gamma_t - gamma_s) of entry (t, s) of this lane's
    // tiles, t = 16w + 4g + i, s = 16j + c16 (s <= t; other entries unused)
    float grow[4] = {0.f, 0.f, 0.f, 0.f}, gcol[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (GATED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) grow[i] = __shfl(gl, 16 * w + 4 * g + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) gcol[j] = __shfl(gl, 16 * j + c16);
    }
    auto decay = [&](int i, int j) { return GATED ? __builtin_amdgcn_exp2f(grow[i] - gcol[j]) : 1.f; };
    if (w == 0) Bt[lane] = lane < nval ? TR::tof(sg.rbeta) : 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * w + 4 * g + i, col = 16 * s2 + c16;
            dPs[row * LT + col] = TR::fromf(col <= row ? pp[s2][i] * decay(i, s2) : 0.f);
            dTs[row * LT + col] = TR::fromf(col <= row ? tt[s2][i] : 0.f);
        }
    __syncthreads();
    // Gram rows of this wave, gm[j][i] = k_t . k_{16j + c16} (t = 16w + 4g + i),
    // and L = their strictly lower part (gated: times the decay factors)
    f32x4 gm[4];
    // gated: this lane's shares of the row sums (rows t) and column sums
    // (columns 16j + c16) of F = dP * P + dL * L, P and L with their decays
    float rsum[4] = {0.f, 0.f, 0.f, 0.f}, csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gm[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kd = 0; kd < NMT; kd += 2)
            gm[j] = TR::mma32(gm[j], ldrow(Ks, L::K, 16 * w + c16, 16 * kd, g), ldrow(Ks, L::K, 16 * w + c16, 16 * kd + 16, g),
                              ldrow(Ks, L::K, 16 * j + c16, 16 * kd, g), ldrow(Ks, L::K, 16 * j + c16, 16 * kd + 16, g));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * w + 4 * g + i, col = 16 * j + c16;
            Ls[t * LT + col] = TR::fromf(col < t ? gm[j][i] * decay(i, j) : 0.f);
        }
    }
    __syncthreads();
    // N = (I + diag(beta) L)^-1 satisfies N = I - T L (T = N diag(beta)), so
    // N^T = I - L^T T^T, an upper triangular product: row block w of it here.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (b >= w) {
#pragma unroll
            for (int k0 = 0; k0 < 64; k0 += 32)
                acc = TR::mma32(acc, TR::ldcol(Ls, LT, k0, 16 * w, g, c16), TR::ldcol(Ls, LT, k0 + 16, 16 * w, g, c16),
                                TR::ldcol(TtS, LT, k0, 16 * b, g, c16), TR::ldcol(TtS, LT, k0 + 16, 16 * b, g, c16));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * w + 4 * g + i, col = 16 * b + c16;
            TsT[row * L::T + col] = TR::fromf((row == col ? 1.f : 0.f) - acc[i]);
        }
    }
    __syncthreads();

    // This wave's token rows t = 16w + 4g + i:
    //   X = N^T dT -> dbeta_a = diag X, Xs = X diag(beta)
    //   G = K K^T (Gram, unscaled)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rb = 0; rb < 4; rb += 2)
            x = TR::mma32(x, ldrow(TsT, L::T, 16 * w + c16, 16 * rb, g), ldrow(TsT, L::T, 16 * w + c16, 16 * rb + 16, g),
                          TR::ldcol(dTs, LT, 16 * rb, 16 * j, g, c16), TR::ldcol(dTs, LT, 16 * rb + 16, 16 * j, g, c16));
        const float bc = Bt[16 * j + c16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (j == w && c16 == 4 * g + i) dba[16 * w + 4 * g + i] = x[i];
            Xs[(16 * w + 4 * g + i) * LT + 16 * j + c16] = TR::fromf(x[i] * bc);
        }
    }
    __syncthreads();
    // dA = -(X diag(beta)) N^T, strictly lower; dbeta_b = sum_j dA_tj G_tj; dL = diag(beta) dA
    float dbb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rb = 0; rb < 4; rb += 2)
            da = TR::mma32(da, ldrow(Xs, LT, 16 * w + c16, 16 * rb, g), ldrow(Xs, LT, 16 * w + c16, 16 * rb + 16, g),
                           TR::ldcol(TsT, L::T, 16 * rb, 16 * j, g, c16), TR::ldcol(TsT, L::T, 16 * rb + 16, 16 * j, g, c16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * w + 4 * g + i, col = 16 * j + c16;
            const float dai = col < t ? -da[i] * decay(i, j) : 0.f; // gated: dA times the decay
            const float m = dai * gm[j][i];
            dbb[i] += m;
            dLs[t * LT + col] = TR::fromf(Bt[t] * dai);
            if constexpr (GATED) {
                const float f = Bt[t] * m; // dL * L
                rsum[i] += f;
                csum[j] += f;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) // sum over the 16 lanes of the row group
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) dbb[i] += __shfl_xor(dbb[i], o, 16);
    __syncthreads();
    sg.store_q(Qs); // N^T and X are no longer read: Q goes over them
    __syncthreads();
    if constexpr (GATED) {
        // F's score part dP * (decayed Q K^T) for this wave's rows (dPs holds dP
        // with the decays), then per token q . dQ (dQ = diag(exp(gamma)) dO S so far)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j > w) break;
            f32x4 qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < NMT; kd += 2)
                qk = TR::mma32(qk, ldrow(Qs, L::K, 16 * w + c16, 16 * kd, g), ldrow(Qs, L::K, 16 * w + c16, 16 * kd + 16, g),
                               ldrow(Ks, L::K, 16 * j + c16, 16 * kd, g), ldrow(Ks, L::K, 16 * j + c16, 16 * kd + 16, g));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * g + i, col = 16 * j + c16;
                const float f = col <= t ? TR::tof(dPs[t * LT + col]) * qk[i] : 0.f;
                rsum[i] += f;
                csum[j] += f;
            }
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) rsum[i] += TR::tof(Qs[(16 * w + 4 * g + i) * L::K + 16 * m + c16]) * dQa[m][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) // over the 16 lanes of the row group
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) rsum[i] += __shfl_xor(rsum[i], o, 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) // over the four row groups
#pragma unroll
            for (int o = 16; o < 64; o <<= 1) csum[j] += __shfl_xor(csum[j], o, 64);
        if (c16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) Rq[16 * w + 4 * g + i] = rsum[i];
        if (g == 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) Cs[64 * w + 16 * j + c16] = csum[j];
    }
    // dQ += dP K;  dK += dP^T Q + (dL + dL^T) K
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int sb = 0; sb < 4; sb += 2) { // 16x16x32 products over token blocks sb, sb + 1
            const F kc0 = TR::ldcol(Ks, L::K, 16 * sb, 16 * m, g, c16), kc1 = TR::ldcol(Ks, L::K, 16 * sb + 16, 16 * m, g, c16);
            dQa[m] = TR::mma32(dQa[m], ldrow(dPs, LT, 16 * w + c16, 16 * sb, g), ldrow(dPs, LT, 16 * w + c16, 16 * sb + 16, g),
                               kc0, kc1);
            dKa[m] = TR::mma32(dKa[m], TR::ldcol(dPs, LT, 16 * sb, 16 * w, g, c16),
                               TR::ldcol(dPs, LT, 16 * sb + 16, 16 * w, g, c16), TR::ldcol(Qs, L::K, 16 * sb, 16 * m, g, c16),
                               TR::ldcol(Qs, L::K, 16 * sb + 16, 16 * m, g, c16));
            dKa[m] = TR::mma32(dKa[m], ldrow(dLs, LT, 16 * w + c16, 16 * sb, g), ldrow(dLs, LT, 16 * w + c16, 16 * sb + 16, g),
                               kc0, kc1);
            dKa[m] = TR::mma32(dKa[m], TR::ldcol(dLs, LT, 16 * sb, 16 * w, g, c16),
                               TR::ldcol(dLs, LT, 16 * sb + 16, 16 * w, g, c16), kc0, kc1);
        }
    E *dkg = reinterpret_cast<E *>(a.dk) + (tok0 + (int64_t)r * kChunk) * sqk + (int64_t)h * DK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * g + i;
        if (t < nval) {
            // dq row: the token itself, or (substeps) the real token, on its last substep only
            int64_t qt = tok0 + (int64_t)r * kChunk + t;
            bool wq = true;
            if constexpr (SUB) {
                const Substep st = substep_at(sg.sb, (uint32_t)(r * kChunk + t));
                qt = st.t;
                wq = st.j == a.nh - 1;
            }
            E *dqg = reinterpret_cast<E *>(a.dq) + qt * sqk + (int64_t)h * DK;
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                if (wq) dqg[16 * m + c16] = TR::fromf(dQa[m][i]);
                dkg[(int64_t)t * sqk + 16 * m + c16] = TR::fromf(dKa[m][i]);
            }
            if (c16 == 0)
                reinterpret_cast<E *>(a.dbeta)[(tok0 + (int64_t)r * kChunk + t) * a.H + h] = TR::fromf(dba[t] + dbb[i]);
        }
    }
    if constexpr (GATED) {
        // d gamma_t = (row t of F) - (column t of F) + q_t . dQ_t - k_t . (a_t + b_t),
        // plus, on the chunk's last prefix sum, sum_t k_t . a_t + exp(gamma_C) <dS', S>
        // (the two make <dS', S'>); dg_t sums d gamma over the chunk's tokens from t on.
        __syncthreads(); // row and column sums complete
        if (w == 0) {
            const int t = lane;
            const float cf = Cs[t] + Cs[64 + t] + Cs[128 + t] + Cs[192 + t];
            float dgam = Rq[t] - cf - xa - xb;
            float sa = xa;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                sa += __shfl_xor(sa, o, 64);
                xs += __shfl_xor(xs, o, 64);
            }
            if (t == 63) dgam += sa + xs;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) { // suffix sum over the lanes
                const float y = __shfl_down(dgam, o, 64);
                dgam += t + o < 64 ? y : 0.f;
            }
            if (t < nval) {
                if constexpr (SUB) { // the decay's gradient is the first substep's
                    const Substep st = substep_at(sg.sb, (uint32_t)(r * kChunk + t));
                    if (st.j == 0) a.dg[st.t * a.H + h] = dgam;
                } else {
                    a.dg[(tok0 + (int64_t)r * kChunk + t) * a.H + h] = dgam;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kimi Delta Attention (KDA) forward, bf16 operands.
//
// "Linear Attention, Visualized", "Kimi Delta Attention (KDA)": the state
// (dv x dk here) first decays per key channel, S <- S Diag(a_t), then the
// delta-rule correction applies. The page's "Complete per-chunk algorithm"
// needs, inside a chunk, products k_l . (lambda[m+1:l] * k_m) whose decay
// differs per channel, so no single row or column scaling of K K^T gives
// them. The kernel therefore runs that algorithm on sub-chunks of 16 tokens
// (the page's exactness holds for every chunk size): with gamma the
// per-channel prefix sums of ln a inside a sub-chunk,
//   Kl = K * exp(gamma),  Ql = Q * exp(gamma)          (factors <= 1; -Kl is
//                                                        stored, so that Y needs
//                                                        no negated copy of S)
//   Kr = K * exp(-gamma)                               (factors >= 1, bounded
//                                                        by 16 tokens of decay)
//   Kf = K * exp(gamma_16 - gamma)                     (factors <= 1)
//   L = Kl Kr^T (strictly lower),  A = Ql Kr^T (lower-inclusive),
//   T = (I + diag(beta) L)^-1 diag(beta)               (DPP forward substitution)
//   Y = V - Kl S^T,  Z = T Y,  O = Ql S^T + A Z,  S <- S Diag(exp(gamma_16)) + Z^T Kf.
// Strong decay: Kr's factor exp(-gamma) is only safe while |gamma| stays
// moderate. A sub-chunk in which some channel's prefix sum leaves
// [-kKdaLim, kKdaLim] (base 2) takes L and A from an exact path instead:
// every entry k_l . (exp(gamma_l - gamma_m) * k_m) (or q_l . ...) is formed
// with the decay factor of the pair itself, which lies in (0, 1] for
// decays, each lane adding its own channels and a 16-lane row reduction
// adding the lanes. Kl, Ql, Kf and exp(gamma_16) only ever carry
// later-minus-earlier differences, so the chain is exact for any decay.
//
// One workgroup of 8 waves per (work item, 64 state rows), in two stages:
//   waves 0-3  (chain) hold 16 state rows each in fp32 registers and run the
//              four sub-chunks of chunk r in order;
//   waves 4-7  (prep) wave 4 + j owns sub-chunk j of chunk r + 1: from its
//              16 tokens' keys, queries and log decays (loaded into registers
//              a chunk ahead, two channels per lane at dk = 128) it forms the
//              prefix sums, the scaled copies, the 16 x 16 blocks L and A
//              (or their exact form) and T, all in its own rows of LDS, so
//              the prep stages need no barrier among themselves.
// One barrier per chunk; the chain reads one half of a double buffer while
// the prep waves fill the other. Wave w and w + 4 share a SIMD.
// ---------------------------------------------------------------------------
// LDS layouts of the KDA kernel. Rows of dk + 16 elements with the 16-byte
// unit index XORed by row bit 3 (okda) keep the 8-byte row reads (16 rows of
// a 16 x 16 block, two lane groups per pass), the transposing reads (8 rows
// x 32 bytes per pass) and the 4-byte writes of the prep waves free of bank
// conflicts; the 16 x 16 blocks use rows of 16 with the same XOR (oblk).
template <int DK> __device__ inline int okda(int r, int c) {
    return r * (DK + 16) + 8 * ((c >> 3) ^ ((r >> 3) & 1)) + (c & 7);
}
__device__ inline int oblk(int r, int c) { return r * 16 + 8 * ((c >> 3) ^ ((r >> 3) & 1)) + (c & 7); }
// KDA rows: dk + 16 elements, the row length of the okda layout.
template <int DK> struct LdKda {
    static constexpr int K = DK + 16;
    static constexpr size_t szK = sizeof(__bf16) * kChunk * K;
};
template <int DK> struct KdaLds {
    using L = LdKda<DK>;
    static constexpr size_t szBlk = 16 * 16 * 2;
    // buffer b: -Kl, Ql, Kf [64][L::K]; exp(gamma_16) fp32 [4][DK]; T^T and A diagonal blocks [4][16][16]
    static constexpr size_t oKL = 0, oQL = L::szK, oKF = 2 * L::szK, oE = 3 * L::szK;
    static constexpr size_t oTB = oE + sizeof(float) * 4 * DK, oPB = oTB + 4 * szBlk, szBuf = oPB + 4 * szBlk;
    // prep only: Kr [64][L::K]; the exact path's row partial sums of one
    // sub-chunk (256 entries x 4 rows of lanes, fp32), over that sub-chunk's
    // own Kr rows where they fit; the fp32 blocks of diag(beta) L [4][16][20]
    static constexpr size_t oKr = 2 * szBuf, szX = sizeof(float) * 256 * 4;
    static constexpr bool kXoverKr = (size_t)16 * L::K * 2 >= szX;
    static constexpr size_t oX = kXoverKr ? oKr : oKr + L::szK;
    static constexpr size_t oAs = kXoverKr ? oKr + L::szK : oX + 4 * szX;
    // chain wave w: its V tile [64 tokens][16 rows] and O^T tile [16 rows][64 tokens]
    // (o64 layout), staging 16-byte loads and 8-byte stores to HBM
    static constexpr size_t oVO = oAs + sizeof(float) * 4 * 16 * 20, szVO = 2 * 64 * 16 * 2;
    static constexpr size_t total = oVO + 4 * szVO;
};
// 64-column bf16 tile with its 8-byte units XORed by row bits 0-3: the
// 8-byte writes of 16 rows at one column and the transposing reads of 8 rows
// at 4 consecutive units are free of bank conflicts.
__device__ inline int okda64(int r, int c) {
    const int s = (((r >> 1) & 3) << 2) | (((r >> 3) & 1) << 1) | (r & 1);
    return r * 64 + 4 * ((c >> 2) ^ s) + (c & 3);
}

// An 8-byte LDS read that the compiler does not pair with a neighbour into
// one ds_read2_b64. The KDA kernel reads the row pieces (16 rows, 4 columns)
// of a tile and the same rows 16 columns on: as a pair those fall on the same
// banks twice over (two-way conflicts), as single reads they do not
// (372.9 -> 359.3 us on the layer workload). The volatile access through an
// LDS-qualified pointer keeps each read whole and in LDS instructions.
__device__ inline bf16x4 ld4_single(const __bf16 *p) {
    return *(const volatile __attribute__((address_space(3))) bf16x4 *)p;
}

// Compile-time loop: f(Int<I>{}) for I = B..E-1 (step indices stay constants).
template <int I> struct Int {
    static constexpr int value = I;
};
template <int B, int E, typename Fn> __device__ inline void static_for(Fn &&f) {
    if constexpr (B < E) {
        f(Int<B>{});
        static_for<B + 1, E>(f);
    }
}

// Prefix-sum bound of the factored path (base 2): Kr = K 2^-gamma and
// Kl = K 2^gamma stay normal and finite in bf16 while |gamma| <= kKdaLim.
constexpr float kKdaLim = 96.f;

// Inclusive sum within each 16-lane row (lanes shifted in from outside the
// row add 0); lane 15 of a row holds the row's total.
__device__ inline float row_scan16(float x) {
    const int zero = 0;
#define DN_ROW_SHR(N)                                                                                          \
    x += __builtin_bit_cast(                                                                                   \
        float, __builtin_amdgcn_update_dpp(zero, __builtin_bit_cast(int, x), 0x110 + (N), 0xF, 0xF, false))
    DN_ROW_SHR(1);
    DN_ROW_SHR(2);
    DN_ROW_SHR(4);
    DN_ROW_SHR(8);
#undef DN_ROW_SHR
    return x;
}

// CPL consecutive channels of one token: a bf16 pair (dk = 128) or one bf16,
// and their log decays; kdv reads channel q as float.
template <int CPL> struct KdaPack;
template <> struct KdaPack<1> {
    using B = __bf16;
    using F = float;
};
template <> struct KdaPack<2> {
    using B = bf16x2;
    using F = float __attribute__((ext_vector_type(2)));
};
__device__ inline float kdv(__bf16 x, int) { return (float)x; }
__device__ inline float kdv(float x, int) { return x; }
__device__ inline float kdv(bf16x2 x, int q) { return (float)x[q]; }
__device__ inline float kdv(float __attribute__((ext_vector_type(2))) x, int q) { return x[q]; }

constexpr int kKdaThreads = 512;

// Compiler-level ordering of LDS accesses within one wave (no instruction).
__device__ inline void lds_order() { asm volatile("" ::: "memory"); }

template <int DK, int DV, bool WO>
__global__ __launch_bounds__(kKdaThreads) void kda_chain_kernel(const ChainArgs a) {
    using E = __bf16;
    using TR = Tr<E>;
    using F = typename TR::F;
    using L = Ld<E, DK>;
    using LY = KdaLds<DK>;
    constexpr int NMT = DK / 16, CPL = DK / 64, RK = DK + 16;
    static_assert(LY::total <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::total];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, c16 = lane & 15;
    // per-lane offsets of the row pieces (c16, 4 g) and of the transposing-read
    // providers (4 g + c16 / 4, 4 (c16 % 4)); a block 16 rows and 16 columns
    // away adds 16 rows of the layout plus 16 (the swizzles keep that affine)
    const int orow = okda<DK>(c16, 4 * g), otr = okda<DK>(4 * g + (c16 >> 2), 4 * (c16 & 3));
    const int brow = oblk(c16, 4 * g), btr = oblk(4 * g + (c16 >> 2), 4 * (c16 & 3));
    auto ld4 = [](const E *p) { return *reinterpret_cast<const bf16x4 *>(p); };
    auto tr4 = [](const E *p) {
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
    };
    // the work item: a token range of one (sequence, head), 64 state rows,
    // where they start and end (dense, packed, or a group of a split sequence)
    const Work wk = decode_work<DK, DV>(a);
    const int h = wk.h, len = wk.len;
    const int64_t tok0 = wk.tok0, sqk = (int64_t)a.H * DK, sv = (int64_t)a.H * DV;
    const int NC = (len + kChunk - 1) / kChunk;
    auto rows_of = [&](int c) { return min(kChunk, len - c * kChunk); };

    if (wave < 4) {
        // ---- chain: state rows 16 w + c16, Sacc[m][i] = S[row0 + 16w + c16][16m + 4g + i] ----
        const int w = wave;
        f32x4 Sacc[NMT];
        state_in<DK>(Sacc, wk, w, g, c16);
        const bool has_v = wk.has_v;
        // this wave's 16 value rows: V loads of 16 bytes (two per lane: token
        // p / 2, half p % 2 of the 32 bytes), O stores of 8 bytes
        const E *vg = reinterpret_cast<const E *>(a.v) + tok0 * sv + (int64_t)h * DV + wk.row0 + 16 * w;
        E *og = WO ? reinterpret_cast<E *>(a.o) + tok0 * sv + (int64_t)h * DV + wk.row0 + 16 * w : nullptr;
        E *Vw = reinterpret_cast<E *>(smem + LY::oVO + w * LY::szVO), *Ow = Vw + 64 * 16;
        bf16x8 vreg[2];
        auto load_v = [&](int c) {
            const int n = rows_of(c);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int p = lane + 64 * s2;
                vreg[s2] = has_v ? *reinterpret_cast<const bf16x8 *>(
                                       vg + (uint32_t)(((int64_t)c * kChunk + min(p >> 1, n - 1)) * sv + 8 * (p & 1)))
                                 : bf16x8{};
            }
        };
        if (NC > 0) load_v(0);
        __syncthreads(); // chunk 0 prepared
        for (int r = 0; r < NC; ++r) {
            const int n = rows_of(r);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) { // V tile of chunk r, rows past the end zero
                const int p = lane + 64 * s2;
                *reinterpret_cast<bf16x8 *>(Vw + 16 * (p >> 1) + 8 * (p & 1)) = (p >> 1) < n ? vreg[s2] : bf16x8{};
            }
            lds_order();
            if (r + 1 < NC) load_v(r + 1);
            const unsigned char *B = smem + (r & 1) * LY::szBuf;
            const E *KLb = reinterpret_cast<const E *>(B + LY::oKL), *QLb = reinterpret_cast<const E *>(B + LY::oQL);
            const E *KFb = reinterpret_cast<const E *>(B + LY::oKF);
            const E *TBb = reinterpret_cast<const E *>(B + LY::oTB), *PBb = reinterpret_cast<const E *>(B + LY::oPB);
            const float *Eb = reinterpret_cast<const float *>(B + LY::oE);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // every LDS operand of the sub-chunk first, so their latency is paid once
                F kl[NMT], ql[NMT], kf[NMT];
                f32x4 ef[NMT];
#pragma unroll
                for (int m = 0; m < NMT; ++m) {
                    kl[m] = ld4_single(KLb + orow + 16 * j * RK + 16 * m);
                    ql[m] = ld4_single(QLb + orow + 16 * j * RK + 16 * m);
                    kf[m] = tr4(KFb + otr + 16 * j * RK + 16 * m);
                    ef[m] = *reinterpret_cast<const f32x4 *>(Eb + j * DK + 16 * m + 4 * g);
                }
                const F tf = tr4(TBb + j * 256 + btr); // row c16 of T_jj
                const F pf = ld4(PBb + j * 256 + brow); // row c16 of A_jj
                const F vf = tr4(Vw + 16 * (16 * j + 4 * g + (c16 >> 2)) + 4 * (c16 & 3)); // V[16j + 4g + e][c16]
                sched_fence();
                F SB[NMT];
#pragma unroll
                for (int m = 0; m < NMT; ++m) SB[m] = TR::cvt(Sacc[m]);
                f32x4 y = widen_bf16(vf);
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NMT; m += 2) { // 16x16x32 products over dk blocks m, m + 1; KL holds -Kl
                    y = TR::mma32(y, kl[m], kl[m + 1], SB[m], SB[m + 1]);
                    o = TR::mma32(o, ql[m], ql[m + 1], SB[m], SB[m + 1]);
                }
                const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
                const F zb = TR::cvt(TR::mma16(z0, tf, TR::cvt(y)));
                o += TR::mma16(z0, pf, zb); // its own accumulator: o comes from 16x16x32 products
                if (WO && has_v) stf(Ow + okda64(c16, 16 * j + 4 * g), TR::cvt(o)); // O^T[c16][16j + 4g + i]
#pragma unroll
                for (int m = 0; m < NMT; ++m) Sacc[m] = TR::mma16(Sacc[m] * ef[m], kf[m], zb);
            }
            if (WO && has_v) { // O rows: lane (g, c16) stores token 16 b + c16, rows 4 g .. 4 g + 3
                lds_order();
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const F x = tr4(Ow + okda64(4 * g + (c16 >> 2), 16 * b + 4 * (c16 & 3)));
                    const int tok = 16 * b + c16;
                    if (tok < n) stf(og + (uint32_t)(((int64_t)r * kChunk + tok) * sv + 4 * g), x);
                }
            }
            lds_order();
            __syncthreads();
        }
        state_out<DK>(Sacc, wk, w, g, c16);
        return;
    }

    // ---- prep: wave 4 + j prepares sub-chunk j, lane l owns channels CPL l .. CPL l + CPL - 1 ----
    const int j = wave - 4, d0 = CPL * lane;
    const E *kg = reinterpret_cast<const E *>(a.k) + tok0 * sqk + (int64_t)h * DK;
    const E *qg = reinterpret_cast<const E *>(a.q) + tok0 * sqk + (int64_t)h * DK;
    const float *gg = a.gk + tok0 * sqk + (int64_t)h * DK;
    const E *bg = reinterpret_cast<const E *>(a.beta) + tok0 * a.H + h;
    E *Kr = reinterpret_cast<E *>(smem + LY::oKr);
    float *Ab = reinterpret_cast<float *>(smem + LY::oAs) + j * 16 * 20; // diag(beta) L of the sub-chunk
    float *Xp = reinterpret_cast<float *>(smem + LY::oX + (LY::kXoverKr ? (size_t)j * 16 * LY::L::K * 2 : j * LY::szX));
    // keys, queries and log decays of the sub-chunk's 16 tokens (this lane's
    // channels, packed), a chunk ahead; beta of token 16 j + c16
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    using KP = typename KdaPack<CPL>::B;
    using GP = typename KdaPack<CPL>::F;
    KP kx[16], qx[16];
    GP gx[16];
    float bx = 0.f;
    auto load = [&](int c, int dd, int cc) {
        const int n = rows_of(c);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t off = (uint32_t)(((int64_t)c * kChunk + min(16 * j + t, n - 1)) * sqk + dd);
            kx[t] = *reinterpret_cast<const KP *>(kg + off);
            qx[t] = *reinterpret_cast<const KP *>(qg + off);
            gx[t] = *reinterpret_cast<const GP *>(gg + off);
        }
        bx = (float)bg[(uint32_t)(((int64_t)c * kChunk + min(16 * j + cc, n - 1)) * a.H)];
    };
    if (NC > 0) load(0, d0, c16);
    // iteration r prepares chunk r + 1 into buffer (r + 1) & 1
    for (int r = -1; r < NC; ++r) {
        const int c = r + 1;
        if (c < NC) {
            // lane coordinates again, opaque to the compiler, so that the
            // offsets derived from them are formed here rather than hoisted out
            // of the loop and kept live (or spilled) across it
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int pg = ln >> 4, pc = ln & 15, pd = CPL * ln;
            const int n = rows_of(c);
            unsigned char *B = smem + (c & 1) * LY::szBuf;
            E *KLb = reinterpret_cast<E *>(B + LY::oKL), *QLb = reinterpret_cast<E *>(B + LY::oQL);
            E *KFb = reinterpret_cast<E *>(B + LY::oKF);
            E *TBj = reinterpret_cast<E *>(B + LY::oTB) + j * 256, *PBj = reinterpret_cast<E *>(B + LY::oPB) + j * 256;
            float *Eb = reinterpret_cast<float *>(B + LY::oE);
            // per-channel prefix sums (base 2); tokens past the end have no decay
            float acc[CPL], gam[16][CPL];
            bool wide = false; // a prefix sum outside the factored path's range
#pragma unroll
            for (int q = 0; q < CPL; ++q) acc[q] = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
#pragma unroll
                for (int q = 0; q < CPL; ++q) {
                    if (16 * j + t < n) acc[q] += kdv(gx[t], q) * 1.44269504088896340736f;
                    gam[t][q] = acc[q];
                    wide |= !(fabsf(acc[q]) <= kKdaLim);
                }
            }
            // exact path for the whole sub-chunk when any of its channels needs it
            const bool exact = __builtin_amdgcn_ballot_w64(wide) != 0;
            float e16[CPL];
#pragma unroll
            for (int q = 0; q < CPL; ++q) e16[q] = __builtin_amdgcn_exp2f(acc[q]);
            // the scaled rows; EXACT and FULL (every token of the sub-chunk
            // inside the sequence) are wave-uniform, so each combination runs
            // without the selects (and, in the factored path, without the
            // third exponential) of the others
            auto scale = [&](auto exact_c, auto full_c) {
                constexpr bool EXACT = decltype(exact_c)::value != 0, FULL = decltype(full_c)::value != 0;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const bool on = FULL || 16 * j + t < n;
                    E a1[CPL], a2[CPL], a3[CPL], a4[CPL];
#pragma unroll
                    for (int q = 0; q < CPL; ++q) {
                        const float kv = on ? kdv(kx[t], q) : 0.f, qv = on ? kdv(qx[t], q) : 0.f;
                        const float el = __builtin_amdgcn_exp2f(gam[t][q]), er = __builtin_amdgcn_exp2f(-gam[t][q]);
                        // exp(gamma_16 - gamma) <= 1: within the factored range the
                        // product of the two factors; beyond it, from the difference itself
                        const float ef = EXACT ? __builtin_amdgcn_exp2f(acc[q] - gam[t][q]) : e16[q] * er;
                        a1[q] = TR::fromf(-(kv * el));
                        a2[q] = TR::fromf(qv * el);
                        a3[q] = TR::fromf(on ? kv * er : 0.f); // er may be infinite past the end (exact path)
                        a4[q] = TR::fromf(kv * ef);
                    }
                    if constexpr (CPL == 2) {
                        const int o = okda<DK>(t, pd) + 16 * j * RK; // t, and so the swizzle, is a constant here
                        *reinterpret_cast<bf16x2 *>(KLb + o) = bf16x2{a1[0], a1[1]};
                        *reinterpret_cast<bf16x2 *>(QLb + o) = bf16x2{a2[0], a2[1]};
                        *reinterpret_cast<bf16x2 *>(Kr + o) = bf16x2{a3[0], a3[1]};
                        *reinterpret_cast<bf16x2 *>(KFb + o) = bf16x2{a4[0], a4[1]};
                    } else {
                        const int o = okda<DK>(t, pd) + 16 * j * RK;
                        KLb[o] = a1[0];
                        QLb[o] = a2[0];
                        Kr[o] = a3[0];
                        KFb[o] = a4[0];
                    }
                }
            };
            const bool full = 16 * j + 15 < n;
            if (exact) {
                if (full) scale(Int<1>{}, Int<1>{});
                else scale(Int<1>{}, Int<0>{});
            } else {
                if (full) scale(Int<0>{}, Int<1>{});
                else scale(Int<0>{}, Int<0>{});
            }
#pragma unroll
            for (int q = 0; q < CPL; ++q) Eb[j * DK + pd + q] = e16[q];
            if (exact) {
                // ln (row rw of 16 lanes, pc) adds its channels of every
                // entry; the 16-ln row scan leaves the row's sum in its ln
                // 15, which stores it: Xp[4 entry + rw]
                float *xp = Xp + (ln >> 4);
                const bool last = pc == 15;
                static_for<0, 16>([&](auto lc) {
                    constexpr int l = decltype(lc)::value;
                    const bool onl = 16 * j + l < n;
                    static_for<0, l + 1>([&](auto mc) {
                        constexpr int m = decltype(mc)::value;
                        float sa = 0.f, sl = 0.f;
#pragma unroll
                        for (int q = 0; q < CPL; ++q) {
                            const float km = 16 * j + m < n ? kdv(kx[m], q) : 0.f;
                            const float t = km * __builtin_amdgcn_exp2f(gam[l][q] - gam[m][q]);
                            sa += (onl ? kdv(qx[l], q) : 0.f) * t;
                            sl += (onl ? kdv(kx[l], q) : 0.f) * t;
                        }
                        sa = row_scan16(sa);
                        if (last) xp[4 * (120 + l * (l + 1) / 2 + m)] = sa; // A entry (l, m)
                        if constexpr (m < l) {
                            sl = row_scan16(sl);
                            if (last) xp[4 * (l * (l - 1) / 2 + m)] = sl; // L entry (l, m)
                        }
                        sched_fence(); // one entry at a time: few registers live
                    });
                });
            }
            const float bt = 16 * j + pc < n ? bx : 0.f; // beta of row 16 j + pc
            // this sub-chunk's registers are consumed: the next chunk's loads go out
            if (c + 1 < NC) load(c + 1, pd, pc);
            // The rows written above are read back by this wave only: LDS keeps
            // a wave's accesses in order, and this keeps the compiler from
            // moving a read of them above the writes (their pointer types differ).
            lds_order();
            if (exact) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int idx = 64 * p + ln, l = idx >> 4, m = idx & 15;
                    float sl = 0.f, sa = 0.f;
                    if (m <= l) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            sa += Xp[4 * (120 + l * (l + 1) / 2 + m) + q];
                            if (m < l) sl += Xp[4 * (l * (l - 1) / 2 + m) + q];
                        }
                    }
                    const float bl = __shfl(bt, l);
                    Ab[l * 20 + m] = m < l ? bl * sl : 0.f;
                    PBj[oblk(l, m)] = TR::fromf(m <= l ? sa : 0.f);
                }
            } else {
                // -L = (-Kl) Kr^T and A = Ql Kr^T over dk, rows 16 j + 4 g + i, columns 16 j + pc
                f32x4 lt = {0.f, 0.f, 0.f, 0.f}, at = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NMT; m += 2) {
                    const int o = okda<DK>(pc, 4 * pg) + 16 * j * RK + 16 * m;
                    const F kr0 = ld4_single(Kr + o), kr1 = ld4_single(Kr + o + 16);
                    lt = TR::mma32(lt, ld4_single(KLb + o), ld4_single(KLb + o + 16), kr0, kr1);
                    at = TR::mma32(at, ld4_single(QLb + o), ld4_single(QLb + o + 16), kr0, kr1);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * pg + i;
                    const float bl = __shfl(bt, row);
                    Ab[row * 20 + pc] = pc < row ? -bl * lt[i] : 0.f;
                    PBj[oblk(row, pc)] = TR::fromf(pc <= row ? at[i] : 0.f);
                }
            }
            lds_order();
            // T = (I + diag(beta) L)^-1 diag(beta): ln pc solves column pc
            // (every ln group the same) and writes row pc of T^T
            float arow[16], x[16];
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(Ab + pc * 20 + 4 * j4);
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * j4 + e] = t[e];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i == pc ? 1.f : 0.f;
            solve_step<0>(x, arow);
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 xv = {x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
                stf(TBj + oblk(pc, 4 * i4), TR::cvt(xv * bt));
            }
        }
        __syncthreads();
    }
}

// One workgroup of 1024 threads: thread t sums the chunk counts of its block
// of sequences, a workgroup scan turns the sums into offsets, and each thread
// then writes the offsets of its block.
__global__ __launch_bounds__(1024) void chunk_base_kernel(const int32_t *cu, int N, int32_t *cb) {
    __shared__ int part[1024];
    const int t = threadIdx.x, per = (N + 1023) / 1024;
    const int b = min(N, t * per), e = min(N, b + per);
    int sum = 0;
    for (int n = b; n < e; ++n) sum += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) { // inclusive scan
        const int x = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int base = t ? part[t - 1] : 0;
    for (int n = b; n < e; ++n) {
        cb[n] = base;
        base += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    }
    if (t == 1023) cb[N] = part[1023];
}

__global__ void fill_kernel(float *p, size_t n, float value) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

template <int DK, int DV> hipError_t launch_bwd_dims(const BwdArgs &a, hipStream_t s) {
    const int units = a.B * a.H * (a.rev_kind == kRevChain ? 1 : a.rev_kind == kRevCpAffine ? a.G - 1 : a.G);
    if (units <= 0 || (!a.cu_seqlens && a.NC <= 0)) return hipSuccess; // varlen: empty sequences still set dS0
    const dim3 cg(units * a.n_tiles);
    if (a.nh > 1)
        hipLaunchKernelGGL((bwd_chain_kernel<DK, DV, true, true>), cg, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<DK, DV, true, false>), cg, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.max_slots <= 0 || a.rev_kind == kRevCpAffine) return hipSuccess; // affine runs write no partial sums
    const dim3 fg((unsigned)a.max_slots);
    if (a.nh > 1)
        hipLaunchKernelGGL((bwd_finish_kernel<DK, DV, true, true>), fg, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((bwd_finish_kernel<DK, DV, true, false>), fg, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_chain(int dtype, int dk, int dv, bool write_o, const ChainArgs &a,
                        hipStream_t stream) {
    if (dtype == 1) return launch_chain_bf16(dk, dv, write_o, a, stream);
    return write_o ? launch_dims_f32<true>(dk, dv, a, stream) : launch_dims_f32<false>(dk, dv, a, stream);
}

hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *cb, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, N, cb);
    return hipGetLastError();
}

hipError_t launch_fill(float *p, size_t n, float value, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n, value);
    return hipGetLastError();
}

template <int DK, int DV> hipError_t launch_kda_dims(bool write_o, const ChainArgs &a, hipStream_t s) {
    const int grid = a.n_units * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    if (write_o)
        hipLaunchKernelGGL((kda_chain_kernel<DK, DV, true>), dim3(grid), dim3(kKdaThreads), 0, s, a);
    else
        hipLaunchKernelGGL((kda_chain_kernel<DK, DV, false>), dim3(grid), dim3(kKdaThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kda(int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_kda_dims<128, 128>(write_o, a, stream);
    if (dk == 128 && dv == 64) return launch_kda_dims<128, 64>(write_o, a, stream);
    if (dk == 64 && dv == 128) return launch_kda_dims<64, 128>(write_o, a, stream);
    if (dk == 64 && dv == 64) return launch_kda_dims<64, 64>(write_o, a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(int dk, int dv, const BwdArgs &a, hipStream_t stream) {
    if (!a.g) return hipErrorInvalidValue; // DeltaNet: launch_bwd_rev, then launch_bwd_grad
    if (dk == 128 && dv == 128) return launch_bwd_dims<128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_bwd_dims<128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_bwd_dims<64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_bwd_dims<64, 64>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_compose_bwd(int dk, int dv, const BwdArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * (dv / 16);
    if (grid <= 0 || a.G < 2) return hipSuccess;
    if (dk == 128 && dv == 128) hipLaunchKernelGGL((compose_bwd_kernel<128, 128>), dim3(grid), dim3(512), 0, stream, a);
    else if (dk == 128 && dv == 64) hipLaunchKernelGGL((compose_bwd_kernel<128, 64>), dim3(grid), dim3(512), 0, stream, a);
    else if (dk == 64 && dv == 128) hipLaunchKernelGGL((compose_bwd_kernel<64, 128>), dim3(grid), dim3(256), 0, stream, a);
    else if (dk == 64 && dv == 64) hipLaunchKernelGGL((compose_bwd_kernel<64, 64>), dim3(grid), dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_compose(int dk, int dv, const ChainArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * (dv / 16);
    if (grid <= 0 || a.G - a.cp_first < 2) return hipSuccess;
    // one wave per output column tile of 16: 64 dk threads
    if (dk == 128 && dv == 128) hipLaunchKernelGGL((compose_kernel<128, 128>), dim3(grid), dim3(512), 0, stream, a);
    else if (dk == 128 && dv == 64) hipLaunchKernelGGL((compose_kernel<128, 64>), dim3(grid), dim3(512), 0, stream, a);
    else if (dk == 64 && dv == 128) hipLaunchKernelGGL((compose_kernel<64, 128>), dim3(grid), dim3(256), 0, stream, a);
    else if (dk == 64 && dv == 64) hipLaunchKernelGGL((compose_kernel<64, 64>), dim3(grid), dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace dn
