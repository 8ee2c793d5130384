// gfx950 bf16 chunk-chain kernel with specialised waves.
//
// One workgroup (8 waves, 512 threads) owns a 64-row slice of one unit's
// state S (dv x dk, acting on column vectors) and walks that unit's chunks in
// order, evaluating per chunk the algorithm of "Linear Attention, Visualized"
// (Haoran Zhang), DeltaNet > "Complete per-chunk algorithm", with S transposed
// as in "Context Parallelism for DeltaNet" (yywangcs), section 2:
//   A  = diag(beta) (K K^T), strictly lower      N = (I + A)^-1,  T = N diag(beta)
//   W  = T K,  U = T V,  P = (Q K^T) lower-inclusive
//   Z  = U - W S^T,  O = Q S^T + P Z,  S <- S + Z^T K.
//
// Wave roles (two waves per SIMD; wave w and w+4 share a SIMD):
//   waves 0-3  consumers: each holds 16 rows of S in fp32 registers and runs
//              Z, O and the state update of chunk r, then U of chunk r+1
//   wave 4     diagonal 16x16 Gram tiles of chunk r+2 and their inverses by
//              forward substitution ("Solving for U": one column per lane,
//              entries of A broadcast along the 16-lane row with DPP)
//   wave 5     off-diagonal Gram tiles of chunk r+2, then the off-diagonal
//              blocks of N by block substitution on the matrix cores
//   waves 6-7  W and P of chunk r+1
//   waves 4-7  also stage K, Q, V and beta from HBM, one iteration ahead
// Each iteration has two barrier-separated phases; the producers run two
// chunks (solve) and one chunk (W, P) ahead of the consumers. LDS rings:
// K x3, Q x2, T^T x2, and one each of W, P, V, so every buffer written in a
// phase is read by nobody in that phase.
//
// Matrix-core layout (16x16x32 bf16, wave64, lane l = 16 g + c, g = l / 16):
// lane l holds row (or column) c of an operand and the 8 contraction slots
// 8g..8g+7; the accumulator's lane l holds D[4g + i][c], i = 0..3. Slots may
// be assigned to any contraction indices as long as both operands agree, so
// the index labels are chosen to make every operand fragment one 16-byte LDS
// read (row fragments) or one transposing read ds_read_b64_tr_b16 per 4 slots
// (column fragments; in a 16-lane group, provider lane p supplies 8 bytes of
// one row and receiver lane i gets element i % 4 of the chunks of providers
// i / 4 + 4e, e = 0..3, so each provider picks its row and 4-column group):
//   * dk index of the state accumulator tile m, lane group g, register i:
//       delta(m, g, i) = 32 (m / 2) + 8 g + 4 (m % 2) + i
//     so a pair of state tiles (2s, 2s+1) gives lane group g the 8
//     consecutive dk values 32 s + 8 g .. +7: W and Q rows are read as one
//     16-byte piece each, straight from their natural row-major layout;
//   * tokens keep their natural order in Z; consecutive Z tiles (2s, 2s+1)
//     give lane group g tokens 32 s + 4 g + e and 32 s + 16 + 4 g + e, so the
//     columns of P are stored in the matching interleaved order.
#include "dn_internal.h"
#include "dn_work.h"

namespace dn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWsThreads = 512;

__device__ inline f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
__device__ inline bf16x4 cvt4(f32x4 x) {
    bf16x4 r;
    r[0] = (__bf16)x[0];
    r[1] = (__bf16)x[1];
    r[2] = (__bf16)x[2];
    r[3] = (__bf16)x[3];
    return r;
}
__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ inline bf16x8 cvt8(f32x4 a, f32x4 b) { return cat8(cvt4(a), cvt4(b)); }
__device__ inline bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x4 ld4(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ inline void st4(__bf16 *p, bf16x4 x) { *reinterpret_cast<bf16x4 *>(p) = x; }
__device__ inline void st8(__bf16 *p, bf16x8 x) { *reinterpret_cast<bf16x8 *>(p) = x; }
// Transposing read: this lane supplies the 8 bytes at p (4 consecutive
// columns of one row); returns this lane's column over the 4 supplied rows.
__device__ inline bf16x4 tr4(const __bf16 *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
}

// Broadcast lane I of each 16-lane row to the whole row (DPP row_newbcast).
template <int I> __device__ inline float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + I, 0xF, 0xF, true));
}
// Column c of (I + A)^-1 for a 16x16 strictly lower A whose row c sits in
// lane c of the 16-lane row: once x_J is final it is removed from every later
// row (right-looking forward substitution).
template <int J> __device__ inline void fwd_subst(float (&x)[16], const float (&arow)[16]) {
    if constexpr (J < 15) {
        const float nxj = -x[J];
#define DN_UPD(I)                                                                                              \
    if constexpr (I > J) x[I] = fmaf(row_bcast<I>(arow[J]), nxj, x[I]);
        DN_UPD(1) DN_UPD(2) DN_UPD(3) DN_UPD(4) DN_UPD(5) DN_UPD(6) DN_UPD(7) DN_UPD(8)
        DN_UPD(9) DN_UPD(10) DN_UPD(11) DN_UPD(12) DN_UPD(13) DN_UPD(14) DN_UPD(15)
#undef DN_UPD
        fwd_subst<J + 1>(x, arow);
    }
}

// LDS layout. Row strides in elements, padded by 16 bytes.
template <int DK> struct WsLds {
    static constexpr int LK = DK + 8;  // K, Q, W: [64][LK] bf16
    static constexpr int L64 = 64 + 8; // T^T, P, V tile: [64][L64] bf16
    static constexpr int LN = 16 + 8;  // N^T of the four diagonal blocks: [64][LN] bf16
    static constexpr int LX = 16 + 4;  // diagonal Gram tiles for the row exchange: [64][LX] fp32
    static constexpr size_t szK = sizeof(__bf16) * 64 * LK;
    static constexpr size_t sz64 = sizeof(__bf16) * 64 * L64;
    static constexpr size_t oK = 0;              // 3 buffers, chunk c in buffer c % 3
    static constexpr size_t oQ = oK + 3 * szK;   // 2 buffers, c % 2
    static constexpr size_t oW = oQ + 2 * szK;   // -W
    static constexpr size_t oT = oW + szK;       // T^T, 2 buffers, c % 2
    static constexpr size_t oP = oT + 2 * sz64;  // P, columns interleaved
    static constexpr size_t oV = oP + sz64;      // V: this workgroup's 64 value columns
    static constexpr size_t oN = oV + sz64;
    static constexpr size_t oX = oN + sizeof(__bf16) * 64 * LN;
    static constexpr size_t oB = oX + sizeof(float) * 64 * LX; // beta ring, 4 x 64 fp32, c % 4
    static constexpr size_t total = oB + sizeof(float) * 4 * 64;
};

// Global -> register -> LDS staging of one chunk, shared by the 256 threads of
// waves 4-7 (pt = 0..255). Loads are unconditional within the chunk: rows past
// the end of the sequence re-read the last valid row and are written as zeros.
template <int DK> struct WsStager {
    static constexpr int KV = DK / 8;          // 16-byte vectors per K / Q row
    static constexpr int NK = 64 * KV / 256;   // K (and Q) vectors per thread
    static constexpr int NV = 64 * 8 / 256;    // vectors per thread of the 64x64 V tile
    static_assert(NK * 256 == 64 * KV, "tiling");
    const __bf16 *kg, *qg, *vg, *bg;
    int64_t sqk, sv;
    int H, len, pt;
    bf16x8 rk[NK], rq[NK], rv[NV];
    __bf16 rb;
    int nk, nq, nv;

    __device__ inline int rows_of(int c) const { return min(kChunk, len - c * kChunk); }
    __device__ inline void load_k(int c) {
        nk = rows_of(c);
        const int64_t base = (int64_t)c * kChunk;
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int v = p * 256 + pt, row = min(v / KV, nk - 1), cv = v % KV;
            rk[p] = ld8g(kg + (base + row) * sqk + 8 * cv);
        }
        if (pt < 64) rb = bg[(base + min(pt, nk - 1)) * H];
    }
    __device__ inline void load_q(int c) {
        nq = rows_of(c);
        const int64_t base = (int64_t)c * kChunk;
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int v = p * 256 + pt, row = min(v / KV, nq - 1), cv = v % KV;
            rq[p] = ld8g(qg + (base + row) * sqk + 8 * cv);
        }
    }
    __device__ inline void load_v(int c) {
        nv = rows_of(c);
        const int64_t base = (int64_t)c * kChunk;
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int v = p * 256 + pt, row = min(v / 8, nv - 1), cv = v % 8;
            rv[p] = ld8g(vg + (base + row) * sv + 8 * cv);
        }
    }
    __device__ inline void write_k(__bf16 *Ks, float *Bs) const {
        const bf16x8 z = {};
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int v = p * 256 + pt, row = v / KV, cv = v % KV;
            st8(Ks + row * WsLds<DK>::LK + 8 * cv, row < nk ? rk[p] : z);
        }
        if (pt < 64) Bs[pt] = pt < nk ? (float)rb : 0.f;
    }
    __device__ inline void write_q(__bf16 *Qs) const {
        const bf16x8 z = {};
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int v = p * 256 + pt, row = v / KV, cv = v % KV;
            st8(Qs + row * WsLds<DK>::LK + 8 * cv, row < nq ? rq[p] : z);
        }
    }
    __device__ inline void write_v(__bf16 *Vs) const {
        const bf16x8 z = {};
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int v = p * 256 + pt, row = v / 8, cv = v % 8;
            st8(Vs + row * WsLds<DK>::L64 + 8 * cv, row < nv ? rv[p] : z);
        }
    }
    __device__ static inline bf16x8 ld8g(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
};

// Shared LDS pointers of one workgroup.
template <int DK> struct WsBufs {
    unsigned char *base;
    __device__ inline __bf16 *K(int c) const { return (__bf16 *)(base + WsLds<DK>::oK + (c % 3) * WsLds<DK>::szK); }
    __device__ inline __bf16 *Q(int c) const { return (__bf16 *)(base + WsLds<DK>::oQ + (c & 1) * WsLds<DK>::szK); }
    __device__ inline __bf16 *W() const { return (__bf16 *)(base + WsLds<DK>::oW); }
    __device__ inline __bf16 *Tt(int c) const { return (__bf16 *)(base + WsLds<DK>::oT + (c & 1) * WsLds<DK>::sz64); }
    __device__ inline __bf16 *P() const { return (__bf16 *)(base + WsLds<DK>::oP); }
    __device__ inline __bf16 *V() const { return (__bf16 *)(base + WsLds<DK>::oV); }
    __device__ inline __bf16 *N() const { return (__bf16 *)(base + WsLds<DK>::oN); }
    __device__ inline float *X() const { return (float *)(base + WsLds<DK>::oX); }
    __device__ inline float *B(int c) const { return (float *)(base + WsLds<DK>::oB) + (c & 3) * 64; }
};

// State rows in and out. Sacc[m][i] = S[row][delta(m, g, i)] for the lane's
// state row (column index c of the accumulator).
template <int DK> __device__ inline int dk_of(int m, int g) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1); }

template <int DK> __device__ inline void ws_state_in(f32x4 (&Sacc)[DK / 16], const Work &wk, int cw, int g, int c16) {
    const int lrow = 16 * cw + c16, srow = wk.row0 + lrow;
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
        const int d0 = dk_of<DK>(m, g);
        if (wk.Sin) {
            Sacc[m] = *reinterpret_cast<const f32x4 *>(wk.Sin + lrow * DK + d0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[m][i] = (wk.identity && d0 + i == srow) ? 1.f : 0.f;
        }
    }
}
template <int DK>
__device__ inline void ws_state_out(const f32x4 (&Sacc)[DK / 16], const Work &wk, int cw, int g, int c16) {
    if (!wk.Sout) return;
    const int lrow = 16 * cw + c16, srow = wk.row0 + lrow;
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
        const int d0 = dk_of<DK>(m, g);
        if (!wk.transposed_out) {
            *reinterpret_cast<f32x4 *>(wk.Sout + lrow * DK + d0) = Sacc[m];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) wk.Sout[(int64_t)(d0 + i) * DK + srow] = Sacc[m][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Consumers (waves 0-3).
// ---------------------------------------------------------------------------
template <int DK, int DV, bool WO>
__device__ void consumer_loop(const ChainArgs &a, const Work &wk, const WsBufs<DK> &bf, int NC, int cw, int g,
                              int c16) {
    using LY = WsLds<DK>;
    constexpr int NMT = DK / 16, NKB = DK / 32;
    const bool has_v = WO || wk.has_v;
    f32x4 Sacc[NMT], Zacc[4];
    ws_state_in<DK>(Sacc, wk, cw, g, c16);
#pragma unroll
    for (int t = 0; t < 4; ++t) Zacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t sv = (int64_t)a.H * DV;
    __bf16 *og = WO ? reinterpret_cast<__bf16 *>(a.o) + wk.tok0 * sv + (int64_t)wk.h * DV + wk.row0 + 16 * cw + 4 * g
                    : nullptr;
    const int kq = c16 >> 2, kr = c16 & 3; // transposing-read provider coordinates

    __syncthreads(); // K(0) staged
    for (int r = -2; r < NC; ++r) {
        // ---------------- phase 1: chain of chunk r
        if (r >= 0) {
            const __bf16 *Wb = bf.W(), *Kb = bf.K(r);
            bf16x8 SB[NKB];
#pragma unroll
            for (int s = 0; s < NKB; ++s) SB[s] = cvt8(Sacc[2 * s], Sacc[2 * s + 1]);
            // Z = U - W S^T  (the W buffer holds -W); Z[t][i] = Z[16t + 4g + i][row c]
            f32x4 Z[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 z = Zacc[t];
#pragma unroll
                for (int s = 0; s < NKB; ++s) z = mfma32(ld8(Wb + (16 * t + c16) * LY::LK + 32 * s + 8 * g), SB[s], z);
                Z[t] = z;
            }
            bf16x8 ZB[2];
            ZB[0] = cvt8(Z[0], Z[1]);
            ZB[1] = cvt8(Z[2], Z[3]);
            f32x4 O[4];
            if constexpr (WO) {
                // O^T = S Q^T + Z^T P^T with the pre-update S; O[t][i] = O[16t + c][row 4g + i]
                const __bf16 *Qb = bf.Q(r), *Pb = bf.P();
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NKB; ++s) o = mfma32(SB[s], ld8(Qb + (16 * t + c16) * LY::LK + 32 * s + 8 * g), o);
#pragma unroll
                    for (int s = 0; s <= t / 2; ++s)
                        o = mfma32(ZB[s], ld8(Pb + (16 * t + c16) * LY::L64 + 32 * s + 8 * g), o);
                    O[t] = o;
                }
            }
            // S^T += K^T Z over the tokens of the chunk
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                const int col = 32 * (m >> 1) + 8 * kr + 4 * (m & 1);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x4 k0 = tr4(Kb + (32 * s + 4 * g + kq) * LY::LK + col);
                    const bf16x4 k1 = tr4(Kb + (32 * s + 16 + 4 * g + kq) * LY::LK + col);
                    Sacc[m] = mfma32(cat8(k0, k1), ZB[s], Sacc[m]);
                }
            }
            if constexpr (WO) {
                const int nval = min(kChunk, wk.len - r * kChunk);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int tok = 16 * t + c16;
                    if (tok < nval) st4(og + ((int64_t)r * kChunk + tok) * sv, cvt4(O[t]));
                }
            }
        }
        __syncthreads();
        // ---------------- phase 2: U of chunk r+1 (T of r+1 and V of r+1 are in LDS)
        if (r + 1 >= 0 && r + 1 < NC) {
            if (has_v) {
                const __bf16 *Tb = bf.Tt(r + 1), *Vb = bf.V();
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s <= t / 2; ++s) {
                        const bf16x4 t0 = tr4(Tb + (32 * s + 4 * g + kq) * LY::L64 + 16 * t + 4 * kr);
                        const bf16x4 t1 = tr4(Tb + (32 * s + 16 + 4 * g + kq) * LY::L64 + 16 * t + 4 * kr);
                        const bf16x4 v0 = tr4(Vb + (32 * s + 4 * g + kq) * LY::L64 + 16 * cw + 4 * kr);
                        const bf16x4 v1 = tr4(Vb + (32 * s + 16 + 4 * g + kq) * LY::L64 + 16 * cw + 4 * kr);
                        u = mfma32(cat8(t0, t1), cat8(v0, v1), u);
                    }
                    Zacc[t] = u; // U[16t + 4g + i][row c]
                }
            }
        }
        __syncthreads();
    }
    ws_state_out<DK>(Sacc, wk, cw, g, c16);
}

// ---------------------------------------------------------------------------
// Producers (waves 4-7). ROLE 0: diagonal solve; 1: off-diagonal Gram and
// block substitution; 2, 3: W and P (halves).
// ---------------------------------------------------------------------------
template <int DK> struct DiagState {};

// Wave 4, phase 1: diagonal Gram tiles G_bb of chunk c, lane group b solves
// block b: lane (b, j) computes column j of N_bb = (I + A_bb)^-1; writes
// N_bb^T (for wave 5) and the diagonal blocks of T^T.
template <int DK>
__device__ inline void diag_solve(const WsBufs<DK> &bf, int c, int g, int c16) {
    using LY = WsLds<DK>;
    constexpr int NKB = DK / 32;
    const __bf16 *Kb = bf.K(c);
    float *X = bf.X();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const bf16x8 kf = ld8(Kb + (16 * b + c16) * LY::LK + 32 * kb + 8 * g);
            acc = mfma32(kf, kf, acc);
        }
        // acc[i] = k_{16b+4g+i} . k_{16b+c} = G_bb[c][4g + i]
        *reinterpret_cast<f32x4 *>(X + (16 * b + c16) * LY::LX + 4 * g) = acc;
    }
    const float br = bf.B(c)[16 * g + c16];
    float arow[16];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(X + (16 * g + c16) * LY::LX + 4 * j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) arow[4 * j4 + e] = (4 * j4 + e < c16) ? t[e] * br : 0.f;
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == c16) ? 1.f : 0.f;
    fwd_subst<0>(x, arow);
    // x[i] = N_gg[i][c]; N^T row 16g + c; T^T row 16g + c, columns 16g..16g+15
    __bf16 *Nr = bf.N() + (16 * g + c16) * LY::LN;
    __bf16 *Tr = bf.Tt(c) + (16 * g + c16) * LY::L64 + 16 * g;
    const f32x4 x0 = {x[0], x[1], x[2], x[3]}, x1 = {x[4], x[5], x[6], x[7]};
    const f32x4 x2 = {x[8], x[9], x[10], x[11]}, x3 = {x[12], x[13], x[14], x[15]};
    st8(Nr, cvt8(x0, x1));
    st8(Nr + 8, cvt8(x2, x3));
    st8(Tr, cvt8(x0 * br, x1 * br));
    st8(Tr + 8, cvt8(x2 * br, x3 * br));
}

// Wave 5, phase 1: off-diagonal Gram tiles of chunk c as bf16 k16 operands,
// A_ac (a > c): lane (g, j) holds A[16a + j][16c + 4g .. +3].
struct OffGram {
    bf16x4 A10, A20, A21, A30, A31, A32;
};
template <int DK> __device__ inline f32x4 gram_tile(const __bf16 *Kb, int a, int cb, int g, int c16) {
    using LY = WsLds<DK>;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb)
        acc = mfma32(ld8(Kb + (16 * cb + c16) * LY::LK + 32 * kb + 8 * g),
                     ld8(Kb + (16 * a + c16) * LY::LK + 32 * kb + 8 * g), acc);
    return acc; // acc[i] = k_{16cb+4g+i} . k_{16a+c} = G[16a + c][16cb + 4g + i]
}
template <int DK> __device__ inline OffGram off_gram(const WsBufs<DK> &bf, int c, int g, int c16) {
    const __bf16 *Kb = bf.K(c);
    const float *Bs = bf.B(c);
    const float b1 = Bs[16 + c16], b2 = Bs[32 + c16], b3 = Bs[48 + c16];
    OffGram o;
    o.A10 = cvt4(gram_tile<DK>(Kb, 1, 0, g, c16) * b1);
    o.A20 = cvt4(gram_tile<DK>(Kb, 2, 0, g, c16) * b2);
    o.A21 = cvt4(gram_tile<DK>(Kb, 2, 1, g, c16) * b2);
    o.A30 = cvt4(gram_tile<DK>(Kb, 3, 0, g, c16) * b3);
    o.A31 = cvt4(gram_tile<DK>(Kb, 3, 1, g, c16) * b3);
    o.A32 = cvt4(gram_tile<DK>(Kb, 3, 2, g, c16) * b3);
    return o;
}

// Wave 5, phase 2: N_ab = -N_aa sum_{c=b}^{a-1} A_ac N_cb for a > b, and
// T_ab = N_ab diag(beta_b) into T^T (row 16b + j, columns 16a + 4g ..).
template <int DK> __device__ inline void off_solve(const WsBufs<DK> &bf, const OffGram &o, int c, int g, int c16) {
    using LY = WsLds<DK>;
    const __bf16 *Ns = bf.N();
    const float *Bs = bf.B(c);
    __bf16 *Tt = bf.Tt(c);
    // B fragments of the diagonal blocks: N_bb[4g + e][c16] = N^T[16b + c16][4g + e]
    const bf16x4 n00 = ld4(Ns + (c16)*LY::LN + 4 * g);
    const bf16x4 n11 = ld4(Ns + (16 + c16) * LY::LN + 4 * g);
    const bf16x4 n22 = ld4(Ns + (32 + c16) * LY::LN + 4 * g);
    // A fragments (rows) of the diagonal blocks: N_aa[c16][4g + e] = N^T[16a + 4g + e][c16]
    const int kq = c16 >> 2, kr = c16 & 3;
    const bf16x4 r11 = tr4(Ns + (16 + 4 * g + kq) * LY::LN + 4 * kr);
    const bf16x4 r22 = tr4(Ns + (32 + 4 * g + kq) * LY::LN + 4 * kr);
    const bf16x4 r33 = tr4(Ns + (48 + 4 * g + kq) * LY::LN + 4 * kr);
    const float be0 = Bs[c16], be1 = Bs[16 + c16], be2 = Bs[32 + c16];
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    auto put = [&](int b, int a, f32x4 nab, float be) { st4(Tt + (16 * b + c16) * LY::L64 + 16 * a + 4 * g, cvt4(nab * be)); };
    // column block 0
    const f32x4 n10 = -mfma16(r11, cvt4(mfma16(o.A10, n00, z)), z);
    const bf16x4 f10 = cvt4(n10);
    const f32x4 n20 = -mfma16(r22, cvt4(mfma16(o.A21, f10, mfma16(o.A20, n00, z))), z);
    const bf16x4 f20 = cvt4(n20);
    const f32x4 n30 = -mfma16(r33, cvt4(mfma16(o.A32, f20, mfma16(o.A31, f10, mfma16(o.A30, n00, z)))), z);
    // column block 1
    const f32x4 n21 = -mfma16(r22, cvt4(mfma16(o.A21, n11, z)), z);
    const bf16x4 f21 = cvt4(n21);
    const f32x4 n31 = -mfma16(r33, cvt4(mfma16(o.A32, f21, mfma16(o.A31, n11, z))), z);
    // column block 2
    const f32x4 n32 = -mfma16(r33, cvt4(mfma16(o.A32, n22, z)), z);
    put(0, 1, n10, be0);
    put(0, 2, n20, be0);
    put(0, 3, n30, be0);
    put(1, 2, n21, be1);
    put(1, 3, n31, be1);
    put(2, 3, n32, be2);
}

// Waves 6-7: W = T K for half of the dk tiles and half of the score tiles of
// chunk c, kept in registers during phase 1 and written in phase 2.
template <int DK> struct WPRegs {
    static constexpr int MT = DK / 32; // dk tiles per wave
    bf16x4 w[MT][4];                   // -W[16nt + c][16mt + 4g ..]
    bf16x4 p[5];                       // score tiles
};

// Score tiles: wave 6 rows blocks {0, 3}, wave 7 blocks {1, 2}.
__device__ constexpr int kPA[2][5] = {{0, 3, 3, 3, 3}, {1, 1, 2, 2, 2}};
__device__ constexpr int kPC[2][5] = {{0, 0, 1, 2, 3}, {0, 1, 0, 1, 2}};

template <int DK, bool WO>
__device__ inline void wp_compute(WPRegs<DK> &R, const WsBufs<DK> &bf, int c, int half, int g, int c16) {
    using LY = WsLds<DK>;
    constexpr int MT = WPRegs<DK>::MT;
    const __bf16 *Kb = bf.K(c), *Tb = bf.Tt(c);
    const int kq = c16 >> 2, kr = c16 & 3;
    // T^T column fragments: lane (g, j) slots = tokens 32s + 16h + 4g + e of column 16nt + j
    bf16x8 tf[4][2];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int s = 0; s <= nt / 2; ++s)
            tf[nt][s] = cat8(tr4(Tb + (32 * s + 4 * g + kq) * LY::L64 + 16 * nt + 4 * kr),
                             tr4(Tb + (32 * s + 16 + 4 * g + kq) * LY::L64 + 16 * nt + 4 * kr));
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
        const int mt = half * MT + mm;
        bf16x8 kf[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
            kf[s] = cat8(tr4(Kb + (32 * s + 4 * g + kq) * LY::LK + 16 * mt + 4 * kr),
                         tr4(Kb + (32 * s + 16 + 4 * g + kq) * LY::LK + 16 * mt + 4 * kr));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s <= nt / 2; ++s) acc = mfma32(kf[s], tf[nt][s], acc);
            // acc[i] = W[16nt + c][16mt + 4g + i]
            R.w[mm][nt] = cvt4(-acc);
        }
    }
    if constexpr (WO) {
        const __bf16 *Qb = bf.Q(c);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int pa = kPA[half][i], pc = kPC[half][i];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                acc = mfma32(ld8(Kb + (16 * pc + c16) * LY::LK + 32 * kb + 8 * g),
                             ld8(Qb + (16 * pa + c16) * LY::LK + 32 * kb + 8 * g), acc);
            // acc[e] = q_{16pa+c} . k_{16pc+4g+e} = P[16pa + c][16pc + 4g + e]
            if (pa == pc) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e > c16) ? 0.f : acc[e];
            }
            R.p[i] = cvt4(acc);
        }
    }
}
template <int DK, bool WO>
__device__ inline void wp_write(const WPRegs<DK> &R, const WsBufs<DK> &bf, int half, int g, int c16) {
    using LY = WsLds<DK>;
    constexpr int MT = WPRegs<DK>::MT;
    __bf16 *Wb = bf.W();
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) st4(Wb + (16 * nt + c16) * LY::LK + 16 * (half * MT + mm) + 4 * g, R.w[mm][nt]);
    if constexpr (WO) {
        __bf16 *Pb = bf.P();
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int pa = kPA[half][i], pc = kPC[half][i];
            // token 16pc + 4g + e sits at column 32 (pc / 2) + 8g + 4 (pc % 2) + e
            st4(Pb + (16 * pa + c16) * LY::L64 + 32 * (pc >> 1) + 8 * g + 4 * (pc & 1), R.p[i]);
        }
    }
}

template <int DK, int DV, bool WO, int ROLE>
__device__ void producer_loop(const ChainArgs &a, const Work &wk, const WsBufs<DK> &bf, int NC, int pt, int g,
                              int c16) {
    const bool has_v = WO || wk.has_v;
    WsStager<DK> st;
    st.sqk = (int64_t)a.H * DK;
    st.sv = (int64_t)a.H * DV;
    st.kg = reinterpret_cast<const __bf16 *>(a.k) + wk.tok0 * st.sqk + (int64_t)wk.h * DK;
    st.qg = reinterpret_cast<const __bf16 *>(a.q) + wk.tok0 * st.sqk + (int64_t)wk.h * DK;
    st.vg = reinterpret_cast<const __bf16 *>(a.v) + wk.tok0 * st.sv + (int64_t)wk.h * DV + wk.row0;
    st.bg = reinterpret_cast<const __bf16 *>(a.beta) + wk.tok0 * a.H + wk.h;
    st.H = a.H;
    st.len = wk.len;
    st.pt = pt;
    st.nk = st.nq = st.nv = 0;
    // prologue: K(0) into LDS; K(1) and Q(0) in flight
    if (NC > 0) {
        st.load_k(0);
        st.write_k(bf.K(0), bf.B(0));
    }
    if (1 < NC) st.load_k(1);
    if (WO && 0 < NC) st.load_q(0);
    __syncthreads();

    OffGram og;
    WPRegs<DK> wr;
    for (int r = -2; r < NC; ++r) {
        // ---------------- phase 1
        if (has_v && r + 1 >= 0 && r + 1 < NC) st.write_v(bf.V());
        if (has_v && r + 2 < NC) st.load_v(r + 2);
        if constexpr (ROLE == 0) {
            if (r + 2 < NC) diag_solve<DK>(bf, r + 2, g, c16);
        } else if constexpr (ROLE == 1) {
            if (r + 2 < NC) og = off_gram<DK>(bf, r + 2, g, c16);
        } else {
            if (r + 1 >= 0 && r + 1 < NC) wp_compute<DK, WO>(wr, bf, r + 1, ROLE - 2, g, c16);
        }
        __syncthreads();
        // ---------------- phase 2
        if constexpr (ROLE == 1) {
            if (r + 2 < NC) off_solve<DK>(bf, og, r + 2, g, c16);
        } else if constexpr (ROLE >= 2) {
            if (r + 1 >= 0 && r + 1 < NC) wp_write<DK, WO>(wr, bf, ROLE - 2, g, c16);
        }
        if (r + 3 < NC) st.write_k(bf.K(r + 3), bf.B(r + 3));
        if (WO && r + 2 < NC) st.write_q(bf.Q(r + 2));
        if (r + 4 < NC) st.load_k(r + 4);
        if (WO && r + 3 < NC) st.load_q(r + 3);
        __syncthreads();
    }
}

template <int DK, int DV, bool WO>
__global__ __launch_bounds__(kWsThreads) void chain_kernel_ws(const ChainArgs a) {
    using LY = WsLds<DK>;
    static_assert(LY::total <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::total];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const Work wk = decode_work<DK, DV>(a);
    const int NC = (wk.len + kChunk - 1) / kChunk;
    const WsBufs<DK> bf{smem};

    // T^T and P: only their lower (P) / upper (T^T) blocks are ever written, so
    // zero both rings once.
    {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 *zt = reinterpret_cast<f32x4 *>(smem + LY::oT);
        constexpr int nvec = (int)((2 * LY::sz64 + LY::sz64) / 16); // T^T x2 and P are contiguous
        for (int i = tid; i < nvec; i += kWsThreads) zt[i] = zero;
    }
    __syncthreads();

    if (wave < 4) {
        consumer_loop<DK, DV, WO>(a, wk, bf, NC, wave, g, c16);
    } else if (wave == 4) {
        producer_loop<DK, DV, WO, 0>(a, wk, bf, NC, tid - 256, g, c16);
    } else if (wave == 5) {
        producer_loop<DK, DV, WO, 1>(a, wk, bf, NC, tid - 256, g, c16);
    } else if (wave == 6) {
        producer_loop<DK, DV, WO, 2>(a, wk, bf, NC, tid - 256, g, c16);
    } else {
        producer_loop<DK, DV, WO, 3>(a, wk, bf, NC, tid - 256, g, c16);
    }
}

template <int DK, int DV, bool WO> hipError_t launch_ws(const ChainArgs &a, hipStream_t s) {
    const int grid = a.n_units * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((chain_kernel_ws<DK, DV, WO>), dim3(grid), dim3(kWsThreads), 0, s, a);
    return hipGetLastError();
}

template <bool WO> hipError_t launch_ws_dims(int dk, int dv, const ChainArgs &a, hipStream_t s) {
    if (dk == 128 && dv == 128) return launch_ws<128, 128, WO>(a, s);
    if (dk == 128 && dv == 64) return launch_ws<128, 64, WO>(a, s);
    if (dk == 64 && dv == 128) return launch_ws<64, 128, WO>(a, s);
    if (dk == 64 && dv == 64) return launch_ws<64, 64, WO>(a, s);
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_chain_bf16(int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t stream) {
    return write_o ? launch_ws_dims<true>(dk, dv, a, stream) : launch_ws_dims<false>(dk, dv, a, stream);
}

} // namespace dn
