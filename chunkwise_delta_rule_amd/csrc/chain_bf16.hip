// gfx950 bf16 chunk-chain kernel with specialised waves.
//
// One workgroup (8 waves, 512 threads) owns a 64-row slice of one unit's
// state S (dv x dk, acting on column vectors) and walks that unit's chunks in
// order, evaluating per chunk the algorithm of "Linear Attention, Visualized"
// (Haoran Zhang), DeltaNet > "Complete per-chunk algorithm", with S transposed
// as in "Context Parallelism for DeltaNet" (yywangcs), section 2:
//   A = diag(beta) (K K^T), strictly lower      N = (I + A)^-1,  T = N diag(beta)
//   P = (Q K^T) lower-inclusive
//   Y = V - K S^T,  Z = T Y,  O = Q S^T + P Z,  S <- S + Z^T K.
// Z is the page's U - W S^T (W = T K, U = T V) with T taken out on the left,
// so neither W nor U is formed: everything that depends on the state is one
// chain of products per 16 state rows, and everything else (Gram tiles, the
// inverse, P) depends only on the chunk and runs ahead of that chain.
//
// Wave roles of the 8-wave, 64-row layout (two waves per SIMD; wave w and
// w+4 share a SIMD; the 12-wave, 32-row and 128-row layouts listed at
// chain_kernel_ws split the same roles differently), iteration r:
//   waves 0-3  consumers: each holds 16 rows of S in fp32 registers and runs
//              Y, Z, O and the state update of chunk r
//   wave 4     all Gram tiles of chunk r+2 from one set of K fragments, and
//              the inverses of the diagonal 16x16 blocks by forward
//              substitution ("Solving for U": one column per lane, entries of
//              A broadcast along the 16-lane row with DPP)
//   wave 5     T of chunk r+1 (off-diagonal blocks by block substitution on
//              the matrix cores, diagonal blocks from wave 4's columns);
//              stages V and beta from HBM
//   waves 6-7  P of chunk r+1, half of the row blocks each; Q goes from HBM
//              straight into their operand registers and on to the Q ring;
//              stage K from HBM
// One barrier per chunk; a buffer written in an iteration is read by nobody
// in that iteration. LDS rings: K x4, Q x2, T^T x2, P x2, V x2, N x2, X x2,
// off-diagonal operands x2, beta x4 (and decay prefix sums x4 when gated).
//
// Gated DeltaNet (same page, "Gated DeltaNet (GDN)" > "Complete per-chunk
// algorithm"). Wave 5 also stages the decay logarithms and turns them into
// in-chunk prefix sums gamma_l (base-2 units, one token per lane). Then
//   A and P take the factor exp(gamma_l - gamma_i) on every unmasked entry,
//   Y = V - diag(exp(gamma)) K S^T, O = diag(exp(gamma)) Q S^T + P Z and
//   S <- exp(gamma_C) S + Z^T diag(exp(gamma_C - gamma)) K.
// The consumers apply the row factors to their accumulators (Y, the Q S^T
// part of O, the state) and to Z before the update; every factor is a
// difference of prefix sums with the later one first, so it lies in (0, 1].
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
//       delta(m, g, i) = 32 (m / 2) + 8 g + 4 ((m + g) % 2) + i
//     so a pair of state tiles (2s, 2s+1) gives lane group g the 8
//     consecutive dk values 32 s + 8 g .. +7 (in one order or the other): K
//     and Q rows are read as one 16-byte piece each from their natural
//     row-major layout, and the transposing reads of K for the state update
//     alternate the two 8-byte halves of each 16-byte unit;
//   * tokens keep their natural order in Y and Z; consecutive tiles (2s,
//     2s+1) give lane group g tokens 32 s + 4 g + e and 32 s + 16 + 4 g + e,
//     so T is read as columns of T^T by transposing reads and P is stored as
//     ready-made operand fragments in that token order.
// LDS rows are unpadded; the 16-byte units of each row are permuted by an XOR
// of a few row bits so that all of the fragment reads above, the 8-byte
// writes of T^T and the staging writes are free of bank conflicts (64 banks
// of 4 bytes; 16 lanes per pass for 16-byte accesses, 32 lanes per pass for
// 8-byte ones).
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
__device__ inline void fence() { __builtin_amdgcn_sched_barrier(0); }
// This lane's index in the wave, formed by two VALU instructions where it is
// used (an asm block the compiler neither hoists nor keeps live).
__device__ inline int lane_id() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
// Lane I of each group of four lanes, broadcast to the four (DPP quad_perm).
template <int I> __device__ inline float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x55 * I, 0xF, 0xF, true));
}
// Lane group g needs a value of the four tokens base + 4g + i (i = 0..3) in
// every lane: lane (g, c) computes the one of token base + 4g + c % 4 and the
// quad spreads them, so each needs one transcendental instead of four.
__device__ inline f32x4 quad_spread(float x) {
    return f32x4{quad_bcast<0>(x), quad_bcast<1>(x), quad_bcast<2>(x), quad_bcast<3>(x)};
}
__device__ inline f32x4 exp2v(f32x4 x) {
    return f32x4{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]), __builtin_amdgcn_exp2f(x[2]),
                 __builtin_amdgcn_exp2f(x[3])};
}

// Compile-time loop: f(Int<I>{}) for I = B..E-1. Long unrolled step lists go
// through this rather than #pragma unroll, whose size limit would otherwise
// leave the step index (and every register array indexed by it) dynamic.
template <int I> struct Int {
    static constexpr int value = I;
};
template <int B, int E, typename F> __device__ inline void static_for(F &&f) {
    if constexpr (B < E) {
        f(Int<B>{});
        static_for<B + 1, E>(f);
    }
}

// acc + a_I * b, where a_I is the value of a in lane I of this lane's 16-lane
// row: one v_fmac_f32 whose first operand is read through DPP row_newbcast.
template <int I> __device__ inline float fmac_bcast(float acc, float a, float b) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(a), "v"(b), "i"(I));
    return acc;
}
// Column c of (I + A)^-1 for a 16x16 strictly lower A whose row c sits in
// lane c of the 16-lane row: once x_J is final it is removed from every later
// row (right-looking forward substitution).
template <int J> __device__ inline void fwd_subst_step(float (&x)[16], const float (&arow)[16]) {
    if constexpr (J < 15) {
        const float nxj = -x[J];
#define DN_UPD(I)                                                                                              \
    if constexpr (I > J) x[I] = fmac_bcast<I>(x[I], arow[J], nxj);
        DN_UPD(1) DN_UPD(2) DN_UPD(3) DN_UPD(4) DN_UPD(5) DN_UPD(6) DN_UPD(7) DN_UPD(8)
        DN_UPD(9) DN_UPD(10) DN_UPD(11) DN_UPD(12) DN_UPD(13) DN_UPD(14) DN_UPD(15)
#undef DN_UPD
        fwd_subst_step<J + 1>(x, arow);
    }
}
__device__ inline void fwd_subst(float (&x)[16], float (&arow)[16]) {
    // DPP reads of a register need two wait states after a VALU write of it:
    // settle all of arow first, then wait once.
    asm volatile("" : "+v"(arow[0]), "+v"(arow[1]), "+v"(arow[2]), "+v"(arow[3]), "+v"(arow[4]), "+v"(arow[5]),
                 "+v"(arow[6]), "+v"(arow[7]), "+v"(arow[8]), "+v"(arow[9]), "+v"(arow[10]), "+v"(arow[11]),
                 "+v"(arow[12]), "+v"(arow[13]), "+v"(arow[14]), "+v"(arow[15]));
    asm volatile("s_nop 1");
    fwd_subst_step<0>(x, arow);
}

// Element offsets inside the LDS buffers. K, Q: [64][DK]; T^T, V tile:
// [64][64]. The 8-element (16-byte) unit u of row r is stored at unit
// u ^ swz(r). LDS reads are served over 64 banks (16 lanes per pass for
// 16-byte reads, 32 for 8-byte and transposing reads) but writes over 32
// banks (8 lanes per pass for 16-byte writes, 16 for 8-byte ones); every
// layout below keeps both free of bank conflicts.
template <int DK> __device__ inline int kswz(int r) {
    // DK = 128: unit bits 0-2 = row bits 0-2 (eight consecutive rows written
    // at one unit hit eight different 32-bank positions) and unit bit 3 =
    // row bit 1 ^ row bit 3 (rows two apart never share a unit pair, which
    // keeps the transposing reads of K^T apart; all 16 rows stay distinct)
    if constexpr (DK == 128)
        return (r & 7) | ((((r >> 1) ^ (r >> 3)) & 1) << 3);
    else // 8 units per row: unit = (b0 ^ b3) ^ 3 b2 ^ 4 b1 for row bits b0..b3
        return ((r ^ (r >> 3)) & 1) ^ (((r >> 2) & 1) * 3) ^ (((r >> 1) & 1) << 2);
}
template <int DK> __device__ inline int koff(int r, int c) { return r * DK + (((c >> 3) ^ kswz<DK>(r)) << 3) + (c & 7); }
__device__ inline int s64swz(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
__device__ inline int s64off(int r, int c) { return r * 64 + (((c >> 3) ^ s64swz(r)) << 3) + (c & 7); }
// T^T: as the 64 x 64 layout, with the two 8-byte halves of every unit
// swapped in odd rows (so that the 8-byte writes of 16 rows at one column
// group fill all 32 write banks).
__device__ inline int ttoff(int r, int c) { return s64off(r, c) ^ (4 * (r & 1)); }
// X ([64][16] fp32, four 16-byte units per row) and N^T ([64][16] bf16, two
// units per row): unit u of row r at u ^ xswz(r) (resp. u ^ nswz(r)).
__device__ inline int xswz(int r) { return ((r >> 2) & 3) ^ (((r >> 1) & 1) << 1); }
__device__ inline int xoff(int r, int u) { return 16 * r + 4 * (u ^ xswz(r)); }
__device__ inline int nswz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
__device__ inline int noff(int r, int c) { return 16 * r + ((((c >> 3) ^ nswz(r)) << 3) | (c & 7)); }
// First dk of the 4-run held by lane group g of state tile m (delta above).
__device__ inline int dk_of(int m, int g) { return 32 * (m >> 1) + 8 * g + 4 * ((m + g) & 1); }
// P operand fragment of token tile t and 32-token block s <= t / 2 (0..5).
__device__ constexpr int pfrag(int t, int s) { return t < 2 ? t : 2 * t - 2 + s; }

// LDS layout (bytes).
template <int DK> struct WsLds {
    static constexpr int LX = 16; // diagonal blocks, one row per lane: [64][LX] fp32
    static constexpr int LN = 16; // N^T of the four diagonal blocks: [64][LN] bf16
    static constexpr size_t szK = sizeof(__bf16) * 64 * DK;
    static constexpr size_t sz64 = sizeof(__bf16) * 64 * 64;
    static constexpr size_t szP = sizeof(__bf16) * 6 * 64 * 8; // six 16x32 operand fragments
    static constexpr size_t szN = sizeof(__bf16) * 64 * LN;
    static constexpr size_t szX = sizeof(float) * 64 * LX;
    static constexpr size_t szA = 6 * 64 * 8;
    static constexpr size_t oK = 0;            // 4 buffers, chunk c in buffer c % 4
    static constexpr size_t oQ = oK + 4 * szK; // 2 buffers, c % 2 (and so on)
    static constexpr size_t oT = oQ + 2 * szK; // T^T
    static constexpr size_t oP = oT + 2 * sz64; // -P as fragments
    static constexpr size_t oV = oP + 2 * szP; // V: this workgroup's 64 value columns
    static constexpr size_t oN = oV + 2 * sz64;
    static constexpr size_t oX = oN + 2 * szN; // Gram rows, then columns of T
    static constexpr size_t oA = oX + 2 * szX; // off-diagonal Gram operands
    static constexpr size_t oB = oA + 2 * szA; // beta ring, 4 x 64 fp32, c % 4
    static constexpr size_t total = oB + sizeof(float) * 4 * 64;
    static constexpr size_t oG = total; // gated: decay prefix sums, 4 x 64 fp32, c % 4
    static constexpr size_t total_gated = oG + sizeof(float) * 4 * 64;
};

// Shared LDS pointers of one workgroup.
template <int DK> struct WsBufs {
    using LY = WsLds<DK>;
    unsigned char *base;
    __device__ inline __bf16 *K(int c) const { return (__bf16 *)(base + LY::oK + (c & 3) * LY::szK); }
    __device__ inline __bf16 *Q(int c) const { return (__bf16 *)(base + LY::oQ + (c & 1) * LY::szK); }
    __device__ inline __bf16 *Tt(int c) const { return (__bf16 *)(base + LY::oT + (c & 1) * LY::sz64); }
    __device__ inline __bf16 *P(int c) const { return (__bf16 *)(base + LY::oP + (c & 1) * LY::szP); }
    __device__ inline __bf16 *V(int c) const { return (__bf16 *)(base + LY::oV + (c & 1) * LY::sz64); }
    // 128-row tiles (no output, so the Q ring is free): V of all 128 value
    // columns as two 64-column halves, half h at Vw(c) + 4096 h
    __device__ inline __bf16 *Vw(int c) const { return (__bf16 *)(base + LY::oQ + (c & 1) * LY::szK); }
    __device__ inline __bf16 *N(int c) const { return (__bf16 *)(base + LY::oN + (c & 1) * LY::szN); }
    __device__ inline float *X(int c) const { return (float *)(base + LY::oX + (c & 1) * LY::szX); }
    __device__ inline __bf16 *A(int c) const { return (__bf16 *)(base + LY::oA + (c & 1) * LY::szA); }
    __device__ inline float *B(int c) const { return (float *)(base + LY::oB) + (c & 3) * 64; }
    __device__ inline float *G(int c) const { return (float *)(base + LY::oG) + (c & 3) * 64; }
};

// Global -> register -> LDS staging. A partial last chunk re-reads its last
// valid row for the missing rows and writes them as zeros. Two register sets
// (chunk parity) keep two chunks in flight.
__device__ inline int rows_of(int len, int c) { return min(kChunk, len - c * kChunk); }

// K by the 128 threads of waves 6-7 (pt = 0..127): thread pt owns the 16-byte
// column piece 8 (pt % KV) of rows pt / KV + RPS p, p = 0..NK-1.
template <int DK> struct KStager {
    static constexpr int KV = DK / 8, NT = 128;
    static constexpr int NK = 64 * KV / NT, RPS = NT / KV;
    static_assert(NK * NT == 64 * KV, "tiling");
    const __bf16 *kt; // row rk0 of chunk 0, column col
    int64_t sqk;
    int len, rk0, col;
    bf16x8 r[2][NK];
    int n[2];
    __device__ inline void init(const __bf16 *kg, int64_t sqk_, int len_, int pt) {
        sqk = sqk_;
        len = len_;
        rk0 = pt / KV;
        col = 8 * (pt % KV);
        kt = kg + rk0 * sqk + col;
        n[0] = n[1] = 0;
    }
    template <int B> __device__ inline void load(int c) {
        n[B] = rows_of(len, c);
        const __bf16 *b = kt + (int64_t)c * kChunk * sqk;
        if (n[B] == kChunk) {
#pragma unroll
            for (int p = 0; p < NK; ++p) r[B][p] = *reinterpret_cast<const bf16x8 *>(b + (int64_t)(RPS * p) * sqk);
        } else {
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int row = min(rk0 + RPS * p, n[B] - 1);
                r[B][p] = *reinterpret_cast<const bf16x8 *>(b + (int64_t)(row - rk0) * sqk);
            }
        }
    }
    template <int B> __device__ inline void write(__bf16 *Ks) const {
        const bf16x8 z = {};
#pragma unroll
        for (int p = 0; p < NK; ++p) {
            const int row = rk0 + RPS * p;
            st8(Ks + koff<DK>(row, col), (n[B] == kChunk || row < n[B]) ? r[B][p] : z);
        }
    }
};

// V tile (64 tokens x NCOL value columns) and beta by the 64 lanes of one
// wave, and beta (and the decay logarithm, when gated) of row l in lane l.
// NCOL = 64: lane l owns the 16-byte piece l % 8 of rows l / 8 + 8 p,
// p = 0..7. NCOL = 32: lane l = 8 a + 4 h + u owns piece u of rows
// (a % 4) + 4 h + 8 (a / 4) + 16 p, p = 0..3, so that each group of 8 lanes
// writes two rows whose swizzles differ in bit 2 (all 32 write banks).
template <int NCOL> struct VStager {
    static constexpr int PPR = NCOL / 8, NV = PPR, RSTEP = 64 / PPR;
    static_assert(NCOL == 64 || NCOL == 32, "tile width");
    const __bf16 *vt, *bt;
    const float *gt; // this head's log decays at real token 0, or nullptr
    SubstepBase sb;  // split of the work's first virtual step
    int64_t sv;
    int H, len, lane, rv0, col;
    bf16x8 r[2][NV];
    __bf16 rb[2];
    float rg[2];
    bool gkeep[2]; // the decay sits on this substep (applied in write_gate, not at the load)
    int n[2], nb[2];
    __device__ inline void init(const __bf16 *vg, const __bf16 *bg, const float *gg, int64_t sv_, int H_, int len_,
                                int lane_) {
        sv = sv_;
        H = H_;
        len = len_;
        lane = lane_;
        if constexpr (NCOL == 64) {
            rv0 = lane / 8;
            col = 8 * (lane % 8);
        } else {
            const int a8 = lane >> 3;
            rv0 = (a8 & 3) + 4 * ((lane >> 2) & 1) + 8 * (a8 >> 2);
            col = 8 * (lane & 3);
        }
        vt = vg + rv0 * sv + col;
        bt = bg;
        gt = gg;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            n[b] = nb[b] = 0;
            rb[b] = (__bf16)0.f;
            rg[b] = 0.f;
            gkeep[b] = false;
#pragma unroll
            for (int p = 0; p < NV; ++p) r[b][p] = bf16x8{};
        }
    }
    template <int B> __device__ inline void load_v(int c) {
        n[B] = rows_of(len, c);
        const __bf16 *b = vt + (int64_t)c * kChunk * sv;
        if (n[B] == kChunk) {
#pragma unroll
            for (int p = 0; p < NV; ++p) r[B][p] = *reinterpret_cast<const bf16x8 *>(b + (int64_t)(RSTEP * p) * sv);
        } else {
#pragma unroll
            for (int p = 0; p < NV; ++p) {
                const int row = min(rv0 + RSTEP * p, n[B] - 1);
                r[B][p] = *reinterpret_cast<const bf16x8 *>(b + (int64_t)(row - rv0) * sv);
            }
        }
    }
    template <int B> __device__ inline void load_beta(int c) {
        nb[B] = rows_of(len, c);
        rb[B] = bt[((int64_t)c * kChunk + min(lane, nb[B] - 1)) * H];
        if (gt) { // the decay sits on the first substep of its real token
            const Substep st = substep_at(sb, (uint32_t)(c * kChunk + min(lane, nb[B] - 1)));
            const float x = gt[st.t * H];
            rg[B] = x;
            gkeep[B] = st.j == 0;
        }
    }
    template <int B> __device__ inline void write_v(__bf16 *Vs) const {
        const bf16x8 z = {};
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int row = rv0 + RSTEP * p;
            st8(Vs + s64off(row, col), (n[B] == kChunk || row < n[B]) ? r[B][p] : z);
        }
    }
    template <int B> __device__ inline void write_beta(float *Bs) const { Bs[lane] = lane < nb[B] ? (float)rb[B] : 0.f; }
    // Inclusive prefix sum of the chunk's decay logarithms over the lanes
    // (token l in lane l), in base-2 units; tokens past the end add nothing.
    template <int B> __device__ inline void write_gate(float *Gs) const {
        Gs[lane] = wave_inclusive_sum(lane < nb[B] && gkeep[B] ? rg[B] * 1.44269504088896340736f : 0.f, lane);
    }
};

// Waves 6-7: the Q rows of two 16-row blocks (wave 6: blocks 0 and 3, wave
// 7: blocks 1 and 2) go from HBM straight into the row fragments of P's
// products (lane (g, j): row 16 b + j, dk 32 kb + 8 g .. +7) and from there
// into the Q ring for the consumers. Rows past the end of the sequence repeat
// its last row; the outputs they feed are never stored. Two register sets
// (chunk parity) keep two chunks in flight.
template <int DK> struct QStage {
    static constexpr int NKB = DK / 32;
    const __bf16 *qt[2]; // row[i] of chunk 0, dk 8 g
    int64_t sqk;
    int len, row[2];
    bf16x8 f[2][2][NKB]; // [set][block][kb]
    __device__ static constexpr int block(int half, int i) { return half ? 1 + i : 3 * i; }
    __device__ inline void init(const __bf16 *qg, int64_t sqk_, int len_, int half, int g, int c16) {
        sqk = sqk_;
        len = len_;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            row[i] = 16 * block(half, i) + c16;
            qt[i] = qg + row[i] * sqk + 8 * g;
        }
    }
    template <int B> __device__ inline void load(int c) {
        const int n = min(kChunk, len - c * kChunk);
        const int64_t off = (int64_t)c * kChunk * sqk;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const __bf16 *b = qt[i] + off + (int64_t)(min(row[i], n - 1) - row[i]) * sqk;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) f[B][i][kb] = *reinterpret_cast<const bf16x8 *>(b + 32 * kb);
        }
    }
    template <int B> __device__ inline void write(__bf16 *Qs, int g) const {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) st8(Qs + koff<DK>(row[i], 32 * kb + 8 * g), f[B][i][kb]);
    }
    // Gated kernels: virtual row M = tok0 + 64 c + row carries the query of
    // its real token on the last substep and zero on the others (qh: this
    // head's query at real token 0, dk 8 g).
    const __bf16 *qh;
    SubstepBase sb; // split of the work's first virtual step
    // The substep test is kept in `keep` and applied by mask_virtual just
    // before the registers are used: a select here would wait on the loads.
    bool keep[2][2];
    template <int B> __device__ inline void load_virtual(int c) {
        const int n = min(kChunk, len - c * kChunk);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const Substep st = substep_at(sb, (uint32_t)(c * kChunk + min(row[i], n - 1)));
            const __bf16 *b = qh + st.t * sqk;
            keep[B][i] = st.j == (int)sb.nh - 1;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) f[B][i][kb] = *reinterpret_cast<const bf16x8 *>(b + 32 * kb);
        }
    }
    template <int B> __device__ inline void mask_virtual() {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) f[B][i][kb] = keep[B][i] ? f[B][i][kb] : bf16x8{};
    }
};

// State rows in and out: Sacc[m][i] = S[row][delta(m, g, i)] for the lane's
// state row (column index c of the accumulator).
template <int DK> __device__ inline void ws_state_in(f32x4 (&Sacc)[DK / 16], const Work &wk, int cw, int g, int c16) {
    const int lrow = 16 * cw + c16, srow = wk.row0 + lrow;
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
        const int d0 = dk_of(m, g);
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
        const int d0 = dk_of(m, g);
        if (!wk.transposed_out) {
            *reinterpret_cast<f32x4 *>(wk.Sout + lrow * DK + d0) = Sacc[m];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) wk.Sout[(int64_t)(d0 + i) * DK + srow] = Sacc[m][i];
        }
    }
}

// Transposing read of the K^T fragment for state tile m (dk delta(m, .)) over
// the 32 tokens 32 s + {4g + e, 16 + 4g + e}; slots in the order of ZB_s.
template <int DK> __device__ inline bf16x8 k_trfrag(const __bf16 *Kb, int m, int s, int g, int c16) {
    const int q = c16 & 3, col = 32 * (m >> 1) + 8 * q + 4 * ((m + q) & 1);
    const int row = 32 * s + 4 * g + (c16 >> 2);
    return cat8(tr4(Kb + koff<DK>(row, col)), tr4(Kb + koff<DK>(row + 16, col)));
}

// ---------------------------------------------------------------------------
// Consumers (waves 0-3).
// ---------------------------------------------------------------------------
// The consumer's work on one chunk as a list of matrix products, each with one
// LDS operand fragment (the other operand is in registers; SB = bf16(-S)):
//   Y  (t, kb):  Y_t += K_{t,kb} SB_kb          4 * DK/32 steps (Y_t starts at V_t)
//   Oq (t, kb):  O_t += SB_kb Q_{t,kb}^T         4 * DK/32 steps (with output)
//   Z  (t, s):   Z_t += T_{t,s} YB_s, s <= t/2   6 steps
//   Op (t, s):   O_t += ZB_s (-P)_{t,s}^T        6 steps (with output)
//   S  (m, s):   S^T_m += K^T_{m,s} ZB_s         2 * DK/16 steps
// O accumulates -O. Half of the Oq steps sit between Y and Z and the other
// half between Z and Op, so the conversions YB = bf16(Y) and ZB = bf16(Z)
// never wait for a product still in flight. Fragments are fetched `depth`
// steps ahead into a rotating register buffer and scheduling fences keep that
// order, so LDS latency hides behind the matrix products in between.
template <int DK, bool WO> struct ChainSteps {
    static constexpr int NKB = DK / 32, NMT = DK / 16;
    static constexpr int nY = 4 * NKB, nOq = WO ? 4 * NKB : 0, nZ = 6, nOp = WO ? 6 : 0, nS = 2 * NMT;
    static constexpr int bOq1 = nY, bZ = bOq1 + nOq / 2, bOq2 = bZ + nZ, bOp = bOq2 + nOq - nOq / 2, bS = bOp + nOp;
    static constexpr int n = bS + nS;
    static constexpr int depth = 8;
    enum { kY, kOq, kZ, kOp, kS };
    static constexpr int kind(int i) {
        return i < bOq1 ? kY : i < bZ ? kOq : i < bOq2 ? kZ : i < bOp ? kOq : i < bS ? kOp : kS;
    }
    static constexpr int idx(int i) {
        return i < bOq1 ? i
               : i < bZ ? i - bOq1
               : i < bOq2 ? i - bZ
               : i < bOp ? i - bOq2 + nOq / 2
               : i < bS ? i - bOp
                        : i - bS;
    }
    // Z / Op step j -> token tile t and 32-token block s (pfrag(tT(j), tS(j)) == j)
    static constexpr int tT(int j) { return j < 2 ? j : j < 4 ? 2 : 3; }
    static constexpr int tS(int j) { return (j == 3 || j == 5) ? 1 : 0; }
};

template <int DK, bool WO> struct ChainSrc {
    const __bf16 *K, *Q, *T, *P;
};

template <int DK, bool WO>
__device__ inline bf16x8 chain_fetch(int i, const ChainSrc<DK, WO> &src, int lane, int g, int c16) {
    using CS = ChainSteps<DK, WO>;
    const int k = CS::kind(i), j = CS::idx(i);
    if (k == CS::kY) return ld8(src.K + koff<DK>(16 * (j / CS::NKB) + c16, 32 * (j % CS::NKB) + 8 * g));
    if (k == CS::kOq) return ld8(src.Q + koff<DK>(16 * (j / CS::NKB) + c16, 32 * (j % CS::NKB) + 8 * g));
    if (k == CS::kZ) {
        // T row 16t + c16 = column of T^T, over tokens 32s + {4g + e, 16 + 4g + e}
        const int t = CS::tT(j), row = 32 * CS::tS(j) + 4 * g + (c16 >> 2), col = 16 * t + 4 * (c16 & 3);
        return cat8(tr4(src.T + ttoff(row, col)), tr4(src.T + ttoff(row + 16, col)));
    }
    if (k == CS::kOp) return ld8(src.P + 512 * j + 8 * lane);
    return k_trfrag<DK>(src.K, j / 2, j % 2, g, c16);
}

__device__ inline f32x4 widen4(bf16x4 v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }

template <int DK, bool WO, bool GATED, int ROWS>
__device__ inline void consumer_chain(const WsBufs<DK> &bf, int r, f32x4 (&Sacc)[DK / 16], __bf16 *og, int64_t sv,
                                      int nval, const SubstepBase &sb, bool has_v, int cw, int lane, int g,
                                      int c16) {
    using CS = ChainSteps<DK, WO>;
    constexpr int D = ROWS == 128 ? (GATED ? 3 : 4) : CS::depth; // 128-row tiles: 128 registers per lane
    const ChainSrc<DK, WO> src{bf.K(r), WO ? bf.Q(r) : nullptr, bf.Tt(r), WO ? bf.P(r) : nullptr};
    bf16x8 SB[CS::NKB], YB[2], ZB[2], ZS[2], buf[D];
    f32x4 Y[4], Z[4], O[4];
    // V_t in the accumulator layout: lane (g, c) gets V[16t + 4g + e][16cw + c]
    bf16x4 vf[4];
    if (has_v) {
        // 128-row tiles: consumers 4-7 read the second 64-column half
        const __bf16 *Vb = ROWS == 128 ? bf.Vw(r) + 4096 * (cw >> 2) : bf.V(r);
        const int vc = ROWS == 128 ? (cw & 3) : cw;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = 32 * s + 4 * g + (c16 >> 2), col = 16 * vc + 4 * (c16 & 3);
            vf[2 * s] = tr4(Vb + s64off(row, col));
            vf[2 * s + 1] = tr4(Vb + s64off(row + 16, col));
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) vf[t] = bf16x4{};
    }
    // Gated: decay factors of the tokens this lane's accumulators touch,
    // formed before the chain so that none of them waits on a product:
    // eg[t][e] = exp(gamma) and ez[t][e] = exp(gamma_C - gamma) of token
    // 16t + 4g + e (rows of Y and Z), eq[t] = exp(gamma) of token 16t + c
    // (columns of O), eC = exp(gamma_C).
    // 128-row tiles (128 registers per lane) keep only the prefix sums gq[t]
    // and form eg and ez where they are used.
    constexpr bool kLazy = ROWS == 128;
    f32x4 eg[4], ez[4];
    float eq[4], gqv[4], gC = 0.f, eC = 1.f;
    if constexpr (GATED) {
        const float *Gs = bf.G(r);
        gC = Gs[kChunk - 1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float gq = Gs[16 * t + 4 * g + (c16 & 3)];
            gqv[t] = gq;
            if constexpr (!kLazy) {
                eg[t] = quad_spread(__builtin_amdgcn_exp2f(gq));
                ez[t] = quad_spread(__builtin_amdgcn_exp2f(gC - gq));
            }
            if constexpr (WO) eq[t] = __builtin_amdgcn_exp2f(Gs[16 * t + c16]);
        }
        eC = __builtin_amdgcn_exp2f(gC);
    }
    static_for<0, D>([&](auto ic) { buf[ic.value] = chain_fetch<DK, WO>(ic.value, src, lane, g, c16); });
    // SB_s slots = dk 32 s + 8 g + 0..7: tiles (2s, 2s+1) hold the low / high
    // half for even g and the other way round for odd g.
    const bool odd = g & 1;
#pragma unroll
    for (int s = 0; s < CS::NKB; ++s) {
        const bf16x4 lo = cvt4(-Sacc[2 * s]), hi = cvt4(-Sacc[2 * s + 1]);
        SB[s] = odd ? cat8(hi, lo) : cat8(lo, hi);
    }
    if constexpr (GATED) { // the decayed state the update adds to
#pragma unroll
        for (int m = 0; m < CS::NMT; ++m) Sacc[m] *= eC;
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        Y[t] = zero; // -K S^T first; V joins before the conversion, so its reads are waited for only there
        Z[t] = zero;
        O[t] = zero;
    }
    fence();
    static_for<0, CS::n>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const bf16x8 f = buf[i % D];
        if constexpr (i + D < CS::n) buf[i % D] = chain_fetch<DK, WO>(i + D, src, lane, g, c16);
        if constexpr (i == CS::bZ) {
            if constexpr (GATED && kLazy) {
#pragma unroll
                for (int t = 0; t < 4; ++t) eg[t] = quad_spread(__builtin_amdgcn_exp2f(gqv[t]));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) Y[t] = GATED ? widen4(vf[t]) + eg[t] * Y[t] : widen4(vf[t]) + Y[t];
            YB[0] = cvt8(Y[0], Y[1]);
            YB[1] = cvt8(Y[2], Y[3]);
        }
        if constexpr (i == CS::bOp) {
            ZB[0] = cvt8(Z[0], Z[1]);
            ZB[1] = cvt8(Z[2], Z[3]);
            if constexpr (GATED) { // rows of Z scaled by exp(gamma_C - gamma_l) for the update
                if constexpr (kLazy) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) ez[t] = quad_spread(__builtin_amdgcn_exp2f(gC - gqv[t]));
                }
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    ZS[s] = cvt8(Z[2 * s] * ez[2 * s], Z[2 * s + 1] * ez[2 * s + 1]);
            }
        }
        fence();
        constexpr int k = CS::kind(i), j = CS::idx(i);
        if constexpr (k == CS::kY) Y[j / CS::NKB] = mfma32(f, SB[j % CS::NKB], Y[j / CS::NKB]);
        if constexpr (k == CS::kOq) O[j / CS::NKB] = mfma32(SB[j % CS::NKB], f, O[j / CS::NKB]);
        if constexpr (k == CS::kZ) Z[CS::tT(j)] = mfma32(f, YB[CS::tS(j)], Z[CS::tT(j)]);
        if constexpr (k == CS::kOp) {
            // gated: the Q S^T part of O tile t is complete; scale its token
            // columns before the first P Z product of the tile
            if constexpr (GATED && CS::tS(j) == 0) O[CS::tT(j)] *= eq[CS::tT(j)];
            O[CS::tT(j)] = mfma32(ZB[CS::tS(j)], f, O[CS::tT(j)]);
        }
        if constexpr (k == CS::kS) Sacc[j / 2] = mfma32(f, GATED ? ZS[j % 2] : ZB[j % 2], Sacc[j / 2]);
        fence();
    });
    if constexpr (WO) {
        // O[t][i] = -O[16t + c][row 4g + i] (rows relative to this wave's 16).
        // Gated kernels: og is the output at real token 0; virtual row
        // 64 r + tok of the work is stored at its real token on the last
        // substep only. The column index comes from the lane id formed here,
        // so that no register holds it across the chain.
        const int cl = lane_id() & 15;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tok = 16 * t + cl;
            if constexpr (GATED) {
                const Substep st = substep_at(sb, (uint32_t)(r * kChunk + tok));
                if (tok < nval && st.j == (int)sb.nh - 1) st4(og + st.t * sv, cvt4(-O[t]));
            } else {
                if (tok < nval) st4(og + (int64_t)tok * sv, cvt4(-O[t]));
            }
        }
    }
}

template <int DK, int DV, bool WO, bool GATED, int ROWS>
__device__ void consumer_loop(const ChainArgs &a, const Work &wk, const WsBufs<DK> &bf, int NC, int cw, int lane,
                              int g, int c16) {
    constexpr int NMT = DK / 16;
    const bool has_v = WO || wk.has_v;
    f32x4 Sacc[NMT];
    ws_state_in<DK>(Sacc, wk, cw, g, c16);
    const int64_t sv = (int64_t)a.H * DV;
    // only dereferenced with output; gated kernels address real tokens from token 0
    __bf16 *og = WO ? reinterpret_cast<__bf16 *>(a.o) + (GATED ? 0 : wk.tok0 * sv) + (int64_t)wk.h * DV + wk.row0 +
                          16 * cw + 4 * g
                    : nullptr;

    const SubstepBase sb = GATED ? substep_base(wk.tok0, a.nh) : SubstepBase{0, 0u, 1u};
    __syncthreads(); // matches the producers' prologue
    for (int r = -3; r < NC; ++r) {
        if (!WO && ROWS != 128 && r >= 0 && wk.Schunks16) { // the state entering chunk r, for the backward pass
            __bf16 *so = wk.Schunks16 + (int64_t)r * DV * DK + (16 * cw + c16) * DK;
#pragma unroll
            for (int m = 0; m < DK / 16; ++m) st4(so + dk_of(m, g), cvt4(Sacc[m]));
        }
        if (r >= 0)
            consumer_chain<DK, WO, GATED, ROWS>(bf, r, Sacc, WO ? og + (GATED ? 0 : (int64_t)r * kChunk * sv) : nullptr,
                                          sv, min(kChunk, wk.len - r * kChunk), sb, has_v, cw, lane, g, c16);
        __syncthreads();
    }
    ws_state_out<DK>(Sacc, wk, cw, g, c16);
}

// ---------------------------------------------------------------------------
// Producers (waves 4-7). ROLE 0: diagonal Gram tiles and solve; 1: T and the
// off-diagonal Gram tiles; 2, 3: P (halves).
// ---------------------------------------------------------------------------

// Row fragments of the four 16-row blocks of a K buffer (slots = dk 32 kb + 8 g ..).
template <int DK> struct KRows {
    bf16x8 f[4][DK / 32];
};
template <int DK, int NB = 4> __device__ inline void k_rows(KRows<DK> &k, const __bf16 *Kb, int g, int c16) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) k.f[b][kb] = ld8(Kb + koff<DK>(16 * b + c16, 32 * kb + 8 * g));
}
// acc[i] = x_{4g + i} . y_{c}, x and y row fragments of two 16-row blocks
template <int DK> __device__ inline f32x4 dot_tile(const bf16x8 (&x)[DK / 32], const bf16x8 (&y)[DK / 32]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) acc = mfma32(x[kb], y[kb], acc);
    return acc;
}

// The Gram tiles of chunk c from K row fragments. gram_diag: the four
// diagonal tiles G_bb go to X(c) (row 16b + j holds G_bb[j][0..15]; G_bb is
// symmetric). gram_off: the off-diagonal tiles A_ac = diag(beta_a) G_ac
// (a > c) go to A(c) as bf16 k16 operands: lane (g, j) holds A[16a + j][16c +
// 4g .. +3], per lane in the order A10, A20, A21, A30, A31, A32. Gated: entry
// (l, i) of A_ac also takes the decay exp(gamma_l - gamma_i). gram_tiles
// (one wave doing both from one set of fragments): the off-diagonal products
// cover the LDS round trip of X before the solve reads it back.
template <int DK> __device__ inline void gram_diag(const KRows<DK> &k, const WsBufs<DK> &bf, int c, int g, int c16) {
    float *X = bf.X(c);
#pragma unroll
    for (int b = 0; b < 4; ++b)
        *reinterpret_cast<f32x4 *>(X + xoff(16 * b + c16, g)) = dot_tile<DK>(k.f[b], k.f[b]);
}
template <int DK, bool GATED>
__device__ inline void gram_off(const KRows<DK> &k, const WsBufs<DK> &bf, int c, int lane, int g, int c16) {
    const float *Bs = bf.B(c);
    const float b1 = Bs[16 + c16], b2 = Bs[32 + c16], b3 = Bs[48 + c16];
    // row factors of A_ac: beta of row token 16a + j, times the decay when gated
    f32x4 s10 = {b1, b1, b1, b1}, s20 = {b2, b2, b2, b2}, s21 = s20, s30 = {b3, b3, b3, b3}, s31 = s30, s32 = s30;
    if constexpr (GATED) {
        // exp(gamma_l - gamma_i) = exp(gamma_l - E_c) exp(E_c - gamma_i), with E_c
        // the prefix sum at the end of column block c: row token l lies after
        // it and column token i in it, so both factors lie in (0, 1]
        const float *Gs = bf.G(c);
        const float g1 = Gs[16 + c16], g2 = Gs[32 + c16], g3 = Gs[48 + c16];
        const float E0 = Gs[15], E1 = Gs[31], E2 = Gs[47];
        const int q = 4 * g + (c16 & 3);
        const f32x4 h0 = quad_spread(__builtin_amdgcn_exp2f(E0 - Gs[q]));
        const f32x4 h1 = quad_spread(__builtin_amdgcn_exp2f(E1 - Gs[16 + q]));
        const f32x4 h2 = quad_spread(__builtin_amdgcn_exp2f(E2 - Gs[32 + q]));
        s10 *= __builtin_amdgcn_exp2f(g1 - E0) * h0;
        s20 *= __builtin_amdgcn_exp2f(g2 - E0) * h0;
        s21 *= __builtin_amdgcn_exp2f(g2 - E1) * h1;
        s30 *= __builtin_amdgcn_exp2f(g3 - E0) * h0;
        s31 *= __builtin_amdgcn_exp2f(g3 - E1) * h1;
        s32 *= __builtin_amdgcn_exp2f(g3 - E2) * h2;
    }
    __bf16 *As = bf.A(c) + 4 * lane;
    // dot_tile(K_c, K_a)[i] = k_{16c+4g+i} . k_{16a+j} = G[16a + j][16c + 4g + i]
    st4(As + 0 * 256, cvt4(dot_tile<DK>(k.f[0], k.f[1]) * s10));
    st4(As + 1 * 256, cvt4(dot_tile<DK>(k.f[0], k.f[2]) * s20));
    st4(As + 2 * 256, cvt4(dot_tile<DK>(k.f[1], k.f[2]) * s21));
    st4(As + 3 * 256, cvt4(dot_tile<DK>(k.f[0], k.f[3]) * s30));
    st4(As + 4 * 256, cvt4(dot_tile<DK>(k.f[1], k.f[3]) * s31));
    st4(As + 5 * 256, cvt4(dot_tile<DK>(k.f[2], k.f[3]) * s32));
}
template <int DK, bool GATED> __device__ inline void gram_tiles(const WsBufs<DK> &bf, int c, int lane, int g, int c16) {
    KRows<DK> k;
    k_rows<DK>(k, bf.K(c), g, c16);
    gram_diag<DK>(k, bf, c, g, c16);
    gram_off<DK, GATED>(k, bf, c, lane, g, c16);
}

// Wave 4, after gram_tiles on the same chunk: lane group b solves diagonal
// block b: lane (b, j) computes column j of N_bb = (I + A_bb)^-1 from row j
// of G_bb (its own row of X); writes N_bb^T (bf16, for wave 5's products)
// and replaces its row of X with column j of T_bb = N_bb beta_j in fp32.
// Gated: entry (j, i) of A_bb also takes the decay exp(gamma_j - gamma_i).
template <int DK, bool GATED> __device__ inline void diag_solve(const WsBufs<DK> &bf, int c, int g, int c16) {
    using LY = WsLds<DK>;
    float *X = bf.X(c);
    const int xr = 16 * g + c16;
    const float br = bf.B(c)[16 * g + c16];
    float arow[16];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        f32x4 t = *reinterpret_cast<const f32x4 *>(X + xoff(xr, j4));
        if constexpr (GATED) {
            const float *Gs = bf.G(c) + 16 * g;
            t *= exp2v(Gs[c16] - *reinterpret_cast<const f32x4 *>(Gs + 4 * j4)); // masked entries unused
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) arow[4 * j4 + e] = (4 * j4 + e < c16) ? t[e] * br : 0.f;
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == c16) ? 1.f : 0.f;
    fwd_subst(x, arow);
    // x[i] = N_gg[i][c]
    __bf16 *N = bf.N(c);
    const f32x4 x0 = {x[0], x[1], x[2], x[3]}, x1 = {x[4], x[5], x[6], x[7]};
    const f32x4 x2 = {x[8], x[9], x[10], x[11]}, x3 = {x[12], x[13], x[14], x[15]};
    st8(N + noff(xr, 0), cvt8(x0, x1));
    st8(N + noff(xr, 8), cvt8(x2, x3));
    *reinterpret_cast<f32x4 *>(X + xoff(xr, 0)) = x0 * br;
    *reinterpret_cast<f32x4 *>(X + xoff(xr, 1)) = x1 * br;
    *reinterpret_cast<f32x4 *>(X + xoff(xr, 2)) = x2 * br;
    *reinterpret_cast<f32x4 *>(X + xoff(xr, 3)) = x3 * br;
}

// Wave 5: T^T of chunk c. Off-diagonal blocks N_ab = -N_aa sum_{c=b}^{a-1}
// A_ac N_cb for a > b on the matrix cores, T_ab = N_ab diag(beta_b) into T^T
// (row 16b + j, columns 16a + 4g ..); diagonal blocks T_bb from X(c).
template <int DK> __device__ inline void off_solve(const WsBufs<DK> &bf, int c, int lane, int g, int c16) {
    using LY = WsLds<DK>;
    const __bf16 *Ns = bf.N(c), *As = bf.A(c) + 4 * lane;
    const float *Bs = bf.B(c), *X = bf.X(c);
    __bf16 *Tt = bf.Tt(c);
    const bf16x4 A10 = ld4(As + 0 * 256), A20 = ld4(As + 1 * 256), A21 = ld4(As + 2 * 256);
    const bf16x4 A30 = ld4(As + 3 * 256), A31 = ld4(As + 4 * 256), A32 = ld4(As + 5 * 256);
    // B fragments of the diagonal blocks: N_bb[4g + e][c16] = N^T[16b + c16][4g + e]
    const bf16x4 n00 = ld4(Ns + noff(c16, 4 * g));
    const bf16x4 n11 = ld4(Ns + noff(16 + c16, 4 * g));
    const bf16x4 n22 = ld4(Ns + noff(32 + c16, 4 * g));
    // A fragments (rows) of the diagonal blocks: N_aa[c16][4g + e] = N^T[16a + 4g + e][c16]
    const int kq = c16 >> 2, kr = c16 & 3;
    const bf16x4 r11 = tr4(Ns + noff(16 + 4 * g + kq, 4 * kr));
    const bf16x4 r22 = tr4(Ns + noff(32 + 4 * g + kq, 4 * kr));
    const bf16x4 r33 = tr4(Ns + noff(48 + 4 * g + kq, 4 * kr));
    const float be0 = Bs[c16], be1 = Bs[16 + c16], be2 = Bs[32 + c16];
    // T^T[16b + c16][16b + 4g + e] = T_bb[4g + e][c16], from row 16b + c16 of X
    f32x4 td[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) td[b] = *reinterpret_cast<const f32x4 *>(X + xoff(16 * b + c16, g));
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    auto put = [&](int b, int a, f32x4 tab) { st4(Tt + ttoff(16 * b + c16, 16 * a + 4 * g), cvt4(tab)); };
    // column block 0
    const f32x4 n10 = -mfma16(r11, cvt4(mfma16(A10, n00, z)), z);
    const bf16x4 f10 = cvt4(n10);
    const f32x4 n20 = -mfma16(r22, cvt4(mfma16(A21, f10, mfma16(A20, n00, z))), z);
    const bf16x4 f20 = cvt4(n20);
    const f32x4 n30 = -mfma16(r33, cvt4(mfma16(A32, f20, mfma16(A31, f10, mfma16(A30, n00, z)))), z);
    // column block 1
    const f32x4 n21 = -mfma16(r22, cvt4(mfma16(A21, n11, z)), z);
    const bf16x4 f21 = cvt4(n21);
    const f32x4 n31 = -mfma16(r33, cvt4(mfma16(A32, f21, mfma16(A31, n11, z))), z);
    // column block 2
    const f32x4 n32 = -mfma16(r33, cvt4(mfma16(A32, n22, z)), z);
#pragma unroll
    for (int b = 0; b < 4; ++b) put(b, b, td[b]);
    put(0, 1, n10 * be0);
    put(0, 2, n20 * be0);
    put(0, 3, n30 * be0);
    put(1, 2, n21 * be1);
    put(1, 3, n31 * be1);
    put(2, 3, n32 * be2);
}

// Waves 6-7: the score tiles of chunk c, wave 6 row blocks {0, 3}, wave 7
// blocks {1, 2}, written as -P operand fragments. Gated: entry (l, i) also
// takes the decay exp(gamma_l - gamma_i).
__device__ constexpr int kPA[2][5] = {{0, 3, 3, 3, 3}, {1, 1, 2, 2, 2}};
__device__ constexpr int kPC[2][5] = {{0, 0, 1, 2, 3}, {0, 1, 0, 1, 2}};
template <int DK, int B, bool GATED>
__device__ inline void p_tiles(const WsBufs<DK> &bf, const QStage<DK> &q, int c, int half, int lane, int g, int c16) {
    const __bf16 *Kb = bf.K(c);
    __bf16 *Pb = bf.P(c) + 8 * lane;
    KRows<DK> k;
    k_rows<DK>(k, Kb, g, c16);
    const float *Gs = bf.G(c);
    bf16x4 p[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int pa = kPA[half][i], pc = kPC[half][i];
        const int qi = half ? pa - 1 : (pa == 3 ? 1 : 0);
        // acc[e] = k_{16pc+4g+e} . q_{16pa+c} = P[16pa + c][16pc + 4g + e]
        f32x4 acc = dot_tile<DK>(k.f[pc], q.f[B][qi]);
        if constexpr (GATED) {
            const float gl = Gs[16 * pa + c16];
            if (pa == pc) { // masked entries are replaced below
                acc *= exp2v(gl - *reinterpret_cast<const f32x4 *>(Gs + 16 * pc + 4 * g));
            } else { // split at the end of column block pc, as for the Gram tiles
                const float E = Gs[16 * pc + 15];
                acc *= __builtin_amdgcn_exp2f(gl - E) *
                       quad_spread(__builtin_amdgcn_exp2f(E - Gs[16 * pc + 4 * g + (c16 & 3)]));
            }
        }
        if (pa == pc) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e > c16) ? 0.f : acc[e];
        }
        p[i] = cvt4(-acc);
    }
    // token 16pc + 4g + e is slot 4 (pc % 2) + e of fragment (pa, pc / 2),
    // lane 16g + c: each fragment is written whole (16 bytes per lane), the
    // tiles right of the diagonal block as zeros
    const bf16x4 z4 = {};
    if (half == 0) {
        st8(Pb + 512 * pfrag(0, 0), cat8(p[0], z4));
        st8(Pb + 512 * pfrag(3, 0), cat8(p[1], p[2]));
        st8(Pb + 512 * pfrag(3, 1), cat8(p[3], p[4]));
    } else {
        st8(Pb + 512 * pfrag(1, 0), cat8(p[0], p[1]));
        st8(Pb + 512 * pfrag(2, 0), cat8(p[2], p[3]));
        st8(Pb + 512 * pfrag(2, 1), cat8(p[4], z4));
    }
}

// Producer roles. A 64-row workgroup has four producer waves:
//   kRoleGram     all Gram tiles of chunk r+2 and the inverses of its diagonal
//                 blocks
//   kRoleVT       V(r+1), beta(r+3) (and the decays) into LDS; T of chunk r+1
//   kRoleKQP0/1   K(r+3) into LDS; Q and half of P of chunk r+1
// A 32-row workgroup has two consumer waves and splits the first two roles
// over four waves, so that each of its six producer waves has less on its
// critical path and the matrix products spread over the SIMDs:
//   kRoleGramDiag diagonal Gram tiles of chunk r+2 and their inverses
//   kRoleGramOff  off-diagonal Gram tiles of chunk r+2
//   kRoleOffSolve T of chunk r+1
//   kRoleV        V(r+1), beta(r+3) (and the decays) into LDS
// A 64-row workgroup of 12 waves (DeltaNet without decay) has four consumers
// and eight producers: the four roles above and the two halves of kRoleKQP
// split into K staging and Q plus P:
//   kRoleK0/1     K(r+3) into LDS (half of the rows each)
//   kRoleQP0/1    Q and half of P of chunk r+1
enum {
    kRoleGram = 0,
    kRoleVT = 1,
    kRoleKQP0 = 2,
    kRoleKQP1 = 3,
    kRoleGramDiag = 4,
    kRoleGramOff = 5,
    kRoleOffSolve = 6,
    kRoleV = 7,
    kRoleK0 = 8,
    kRoleK1 = 9,
    kRoleQP0 = 10,
    kRoleQP1 = 11,
    kRoleV1 = 12 // 128-row tiles: the second 64-column half of V (kRoleV stages the first and beta)
};

template <int DK, int DV, bool WO, bool GATED, int ROLE, int ROWS>
__device__ void producer_loop(const ChainArgs &a, const Work &wk, const WsBufs<DK> &bf, int NC, int g, int c16) {
    constexpr bool kGramDiag = ROLE == kRoleGram || ROLE == kRoleGramDiag;
    constexpr bool kGramOff = ROLE == kRoleGram || ROLE == kRoleGramOff;
    constexpr bool kStageV = ROLE == kRoleVT || ROLE == kRoleV || ROLE == kRoleV1;
    constexpr bool kStageBeta = ROLE == kRoleVT || ROLE == kRoleV;
    constexpr int kVHalf = ROLE == kRoleV1 ? 1 : 0;
    static_assert(ROWS == 128 || ROLE != kRoleV1, "second V half: 128-row tiles only");
    constexpr bool kOffSolve = ROLE == kRoleVT || ROLE == kRoleOffSolve;
    constexpr bool kStageK = ROLE == kRoleKQP0 || ROLE == kRoleKQP1 || ROLE == kRoleK0 || ROLE == kRoleK1;
    constexpr bool kQP = ROLE == kRoleKQP0 || ROLE == kRoleKQP1 || ROLE == kRoleQP0 || ROLE == kRoleQP1;
    constexpr int half = (ROLE == kRoleKQP1 || ROLE == kRoleK1 || ROLE == kRoleQP1) ? 1 : 0;
    const bool has_v = WO || wk.has_v;
    const int lane = 16 * g + c16;
    const int64_t sqk = (int64_t)a.H * DK, sv = (int64_t)a.H * DV;
    KStager<DK> ks;
    VStager<(ROWS == 128 ? 64 : ROWS)> vs;
    QStage<DK> q;
    if constexpr (kStageV) {
        vs.init(reinterpret_cast<const __bf16 *>(a.v) + wk.tok0 * sv + (int64_t)wk.h * DV + wk.row0 + 64 * kVHalf,
                reinterpret_cast<const __bf16 *>(a.beta) + wk.tok0 * a.H + wk.h,
                GATED ? a.g + wk.h : nullptr, sv, a.H, wk.len, lane);
        if constexpr (GATED) vs.sb = substep_base(wk.tok0, a.nh);
    }
    if constexpr (kStageK)
        ks.init(reinterpret_cast<const __bf16 *>(a.k) + wk.tok0 * sqk + (int64_t)wk.h * DK, sqk, wk.len,
                64 * half + lane);
    if constexpr (kQP) {
        if constexpr (WO)
            q.init(reinterpret_cast<const __bf16 *>(a.q) + wk.tok0 * sqk + (int64_t)wk.h * DK, sqk, wk.len, half, g,
                   c16);
        if constexpr (WO && GATED) {
            q.qh = reinterpret_cast<const __bf16 *>(a.q) + (int64_t)wk.h * DK + 8 * g;
            q.sb = substep_base(wk.tok0, a.nh);
        }
    }
    if (NC > 0) { // K(0), K(1), beta(0), beta(1) are written in the first two iterations
        if constexpr (kStageK) {
            ks.template load<0>(0);
            ks.template load<1>(min(1, NC - 1));
        }
        if constexpr (kStageBeta) {
            vs.template load_beta<0>(0);
            vs.template load_beta<1>(min(1, NC - 1));
        }
    }
    __syncthreads();
    if (NC == 0) { // no chunks: the same barriers as the consumers' three iterations
#pragma unroll
        for (int i = 0; i < 3; ++i) __syncthreads();
        return;
    }

    // Iteration r: chunks as in the role list above.
    // Every staging copy comes from registers loaded two iterations before
    // (register set = chunk parity; R = r & 1 is a template argument, so the
    // loop runs two iterations per trip) and is replaced by the loads of the
    // chunk two further on. Staging is unconditional (chunk indices clamped
    // to the sequence): copies outside it land in ring slots that are never
    // read, and straight-line loads let every wait count only the loads it
    // needs.
    const int last = NC - 1;
    auto iteration = [&](int r, auto rpar) {
        constexpr int S = 1 - decltype(rpar)::value; // set of chunks r+1, r+3, r+5
        if constexpr (ROLE == kRoleGram) {
            if (r + 2 >= 0 && r + 2 < NC) {
                gram_tiles<DK, GATED>(bf, r + 2, lane, g, c16);
                diag_solve<DK, GATED>(bf, r + 2, g, c16);
            }
        } else if constexpr (kGramDiag || kGramOff) {
            if (r + 2 >= 0 && r + 2 < NC) {
                KRows<DK> k;
                k_rows<DK>(k, bf.K(r + 2), g, c16);
                if constexpr (kGramDiag) {
                    gram_diag<DK>(k, bf, r + 2, g, c16);
                    diag_solve<DK, GATED>(bf, r + 2, g, c16);
                } else {
                    gram_off<DK, GATED>(k, bf, r + 2, lane, g, c16);
                }
            }
        }
        if constexpr (kStageV) {
            if (has_v) vs.template write_v<S>(ROWS == 128 ? bf.Vw(r + 1) + 4096 * kVHalf : bf.V(r + 1));
            if constexpr (kStageBeta) {
                vs.template write_beta<S>(bf.B(r + 3));
                if constexpr (GATED) vs.template write_gate<S>(bf.G(r + 3));
            }
            if (has_v) vs.template load_v<S>(min(max(r + 3, 0), last));
            if constexpr (kStageBeta) vs.template load_beta<S>(min(r + 5, last));
        }
        if constexpr (kOffSolve) {
            if (r + 1 >= 0 && r + 1 < NC) {
                off_solve<DK>(bf, r + 1, lane, g, c16);
                if constexpr (!WO) {
                    // for the backward pass: T^T of the chunk, row-major, from this
                    // wave's own LDS writes (its blocks are complete here)
                    if (wk.Tchunks) {
                        const __bf16 *Tt = bf.Tt(r + 1);
                        __bf16 *dst = wk.Tchunks + (int64_t)(r + 1) * kChunk * kChunk;
#pragma unroll
                        for (int p = 0; p < 8; ++p) {
                            const int piece = 64 * p + lane, row = piece >> 3, c8 = piece & 7;
                            bf16x8 x = ld8(Tt + s64off(row, 8 * c8));
                            if (row & 1) x = __builtin_shufflevector(x, x, 4, 5, 6, 7, 0, 1, 2, 3);
                            st8(dst + row * kChunk + 8 * c8, x);
                        }
                    }
                }
            }
        }
        if constexpr (kStageK) {
            ks.template write<S>(bf.K(r + 3));
            ks.template load<S>(min(r + 5, last));
        }
        if constexpr (kQP) {
            if constexpr (WO) {
                if (r + 1 >= 0 && r + 1 < NC) {
                    if constexpr (GATED) q.template mask_virtual<S>();
                    q.template write<S>(bf.Q(r + 1), g);
                    p_tiles<DK, S, GATED>(bf, q, r + 1, half, lane, g, c16);
                }
            }
            if constexpr (WO) {
                if constexpr (GATED)
                    q.template load_virtual<S>(min(max(r + 3, 0), last));
                else
                    q.template load<S>(min(max(r + 3, 0), last));
            }
        }
        __syncthreads();
    };
    for (int r = -3; r < NC; r += 2) { // r odd
        iteration(r, Int<1>{});
        if (r + 1 < NC) iteration(r + 1, Int<0>{});
    }
}

// Wave w runs on SIMD w % 4. Layouts (NW waves, ROWS state rows):
//   NW = 8,  ROWS = 64: waves 0-3 consumers; 4-7 kRoleGram, kRoleVT,
//            kRoleKQP0, kRoleKQP1
//   NW = 12, ROWS = 64 (forward with output, no decay): waves 0-3
//            consumers; 4-11 kRoleOffSolve, kRoleGramOff, kRoleK0, kRoleV,
//            kRoleGramDiag, kRoleK1, kRoleQP0, kRoleQP1 (matrix products of
//            about 2.6-2.7k cycles per chunk on every SIMD)
//   NW = 8,  ROWS = 32: waves 0-1 consumers; 2-7 kRoleGramDiag,
//            kRoleGramOff, kRoleOffSolve, kRoleV, kRoleKQP0, kRoleKQP1 (the
//            consumers share their SIMDs with the lightest producers)
//   NW = 15, ROWS = 128 (context-parallel transitions, no output,
//            dk = dv = 128): waves 0-7 consumers; 8-14 kRoleGramOff,
//            kRoleGramDiag, kRoleOffSolve, kRoleV, kRoleK0, kRoleK1, kRoleV1.
//            One tile covers all value rows of Q_g or all key rows of P_g,
//            so the chunk's Gram tiles, inverses and T are formed once for
//            128 state rows instead of once per 64
// Twelve waves leave 168 registers per lane, too few for the consumers of
// the decayed kernels, which keep the 8-wave layout; fifteen leave 128.
template <int DK, int DV, bool WO, bool GATED, int ROWS, int NW>
__global__ __launch_bounds__(NW * 64) void chain_kernel_ws(const ChainArgs a) {
    using LY = WsLds<DK>;
    constexpr size_t kLds = GATED ? LY::total_gated : LY::total;
    static_assert(kLds <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const Work wk = decode_work<DK, DV, ROWS>(a);
    const int NC = (wk.len + kChunk - 1) / kChunk;
    const WsBufs<DK> bf{smem};

    // T^T and P: only the blocks of T's lower triangle and P's lower-inclusive
    // triangle are ever written, so zero both rings once.
    {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 *zt = reinterpret_cast<f32x4 *>(smem + LY::oT);
        constexpr int nvec = (int)((2 * LY::sz64 + 2 * LY::szP) / 16); // T^T x2 and P x2 are contiguous
        for (int i = tid; i < nvec; i += NW * 64) zt[i] = zero;
    }
    __syncthreads();

    if constexpr (ROWS == 128) {
        static_assert(NW == 15 && !WO && DK == 128 && DV == 128, "128-row tiles");
        if (wave < 8) {
            consumer_loop<DK, DV, WO, GATED, ROWS>(a, wk, bf, NC, wave, lane, g, c16);
        } else if (wave == 8) {
            producer_loop<DK, DV, WO, GATED, kRoleGramOff, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 9) {
            producer_loop<DK, DV, WO, GATED, kRoleGramDiag, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 10) {
            producer_loop<DK, DV, WO, GATED, kRoleOffSolve, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 11) {
            producer_loop<DK, DV, WO, GATED, kRoleV, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 12) {
            producer_loop<DK, DV, WO, GATED, kRoleK0, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 13) {
            producer_loop<DK, DV, WO, GATED, kRoleK1, ROWS>(a, wk, bf, NC, g, c16);
        } else {
            producer_loop<DK, DV, WO, GATED, kRoleV1, ROWS>(a, wk, bf, NC, g, c16);
        }
    } else if constexpr (NW == 12) {
        static_assert(ROWS == 64, "tile rows");
        if (wave < 4) {
            consumer_loop<DK, DV, WO, GATED, ROWS>(a, wk, bf, NC, wave, lane, g, c16);
        } else if (wave == 4) {
            producer_loop<DK, DV, WO, GATED, kRoleOffSolve, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 5) {
            producer_loop<DK, DV, WO, GATED, kRoleGramOff, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 6) {
            producer_loop<DK, DV, WO, GATED, kRoleK0, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 7) {
            producer_loop<DK, DV, WO, GATED, kRoleV, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 8) {
            producer_loop<DK, DV, WO, GATED, kRoleGramDiag, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 9) {
            producer_loop<DK, DV, WO, GATED, kRoleK1, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 10) {
            producer_loop<DK, DV, WO, GATED, kRoleQP0, ROWS>(a, wk, bf, NC, g, c16);
        } else {
            producer_loop<DK, DV, WO, GATED, kRoleQP1, ROWS>(a, wk, bf, NC, g, c16);
        }
    } else if constexpr (ROWS == 64) {
        static_assert(NW == 8, "waves");
        if (wave < 4) {
            consumer_loop<DK, DV, WO, GATED, ROWS>(a, wk, bf, NC, wave, lane, g, c16);
        } else if (wave == 4) {
            producer_loop<DK, DV, WO, GATED, kRoleGram, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 5) {
            producer_loop<DK, DV, WO, GATED, kRoleVT, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 6) {
            producer_loop<DK, DV, WO, GATED, kRoleKQP0, ROWS>(a, wk, bf, NC, g, c16);
        } else {
            producer_loop<DK, DV, WO, GATED, kRoleKQP1, ROWS>(a, wk, bf, NC, g, c16);
        }
    } else {
        static_assert(ROWS == 32 && NW == 8, "tile rows");
        if (wave < 2) {
            consumer_loop<DK, DV, WO, GATED, ROWS>(a, wk, bf, NC, wave, lane, g, c16);
        } else if (wave == 2) {
            producer_loop<DK, DV, WO, GATED, kRoleGramDiag, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 3) {
            producer_loop<DK, DV, WO, GATED, kRoleGramOff, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 4) {
            producer_loop<DK, DV, WO, GATED, kRoleOffSolve, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 5) {
            producer_loop<DK, DV, WO, GATED, kRoleV, ROWS>(a, wk, bf, NC, g, c16);
        } else if (wave == 6) {
            producer_loop<DK, DV, WO, GATED, kRoleKQP0, ROWS>(a, wk, bf, NC, g, c16);
        } else {
            producer_loop<DK, DV, WO, GATED, kRoleKQP1, ROWS>(a, wk, bf, NC, g, c16);
        }
    }
}

// ---------------------------------------------------------------------------
// Reverse chain of the DeltaNet backward pass.
//
// The pages give no backward pass; this is the chain rule on the per-chunk
// algorithm above. For a chunk with upstream dO and dS' (the gradient of the
// state after the chunk):
//   dZ = P^T dO + K dS'^T,  dY = T^T dZ,  dV = dY,
//   dS = dS' + dO^T Q - dY^T K.
// The state gradient enters only through K dS'^T, so this is the forward's
// chain run backwards with T^T for T, P^T dO for V and one more product
// (dO^T Q) in the update. Rows of dS (value index) are independent, so 64-row
// tiles split it as in the forward. T^T of each chunk comes from the forward
// pass; P is formed here. The kernel writes dV, the dS' of every chunk
// (bf16, for the chunk-parallel gradient kernel) and dS0.
//
// Waves: 0-3 carry 16 rows of dS each in fp32 registers (accumulator layout
// of the forward's state, G[m][i] = dS[row][delta(m, g, i)]); wave 4 stages
// T^T, wave 5 the dO tile, waves 6-7 stage K and Q and form P^T as ready-made
// operand fragments. Step i of the loop is chunk NC - 1 - i; one barrier per
// step; producers work one step (T^T, dO, Q, P^T) or two (K) ahead.
// ---------------------------------------------------------------------------
template <int DK> struct RevLds {
    static constexpr size_t szK = sizeof(__bf16) * 64 * DK;
    static constexpr size_t sz64 = sizeof(__bf16) * 64 * 64;
    static constexpr size_t szP = sizeof(__bf16) * 6 * 64 * 8;
    static constexpr size_t oK = 0;             // K x3, step i in buffer (i + 3) % 3
    static constexpr size_t oQ = oK + 3 * szK;  // Q x2 (step parity)
    static constexpr size_t oT = oQ + 2 * szK;  // T^T x2, row-major (64 x 64 layout)
    static constexpr size_t oP = oT + 2 * sz64; // P^T operand fragments x2
    static constexpr size_t oD = oP + 2 * szP;  // dO tile x2 (64 tokens x 64 values)
    static constexpr size_t total = oD + 2 * sz64;
};
template <int DK> struct RevBufs {
    using LY = RevLds<DK>;
    unsigned char *base;
    __device__ inline __bf16 *K(int i) const { return (__bf16 *)(base + LY::oK + ((i + 3) % 3) * LY::szK); }
    __device__ inline __bf16 *Q(int i) const { return (__bf16 *)(base + LY::oQ + (i & 1) * LY::szK); }
    __device__ inline __bf16 *Tt(int i) const { return (__bf16 *)(base + LY::oT + (i & 1) * LY::sz64); }
    __device__ inline __bf16 *P(int i) const { return (__bf16 *)(base + LY::oP + (i & 1) * LY::szP); }
    __device__ inline __bf16 *D(int i) const { return (__bf16 *)(base + LY::oD + (i & 1) * LY::sz64); }
};

// What one reverse-chain workgroup works on: a (sequence, head) unit and 64
// value rows, its token range and its chunk slots.
struct RevWork {
    int64_t tok0, slot0, su;
    int len, h, row0;
    const float *gin; // rows of the gradient at the end of the token range, or nullptr (zero)
    float *gout;      // rows of the gradient at its start, or nullptr
    bool store;       // write dv and the dS' of every chunk
};
// Work units of the reverse chain: (sequence, head) units, or (b, h, group)
// for the context-parallel kinds (groups 1..G-1 for kRevCpAffine, all G for
// kRevCpRun).
__device__ inline int rev_units(const BwdArgs &a) {
    return a.rev_kind == kRevChain ? a.B * a.H : a.B * a.H * (a.rev_kind == kRevCpAffine ? a.G - 1 : a.G);
}
template <int DK, int DV> __device__ inline RevWork rev_work(const BwdArgs &a) {
    int u, tau;
    map_block(blockIdx.x, rev_units(a), a.n_tiles, u, tau); // the tiles of a unit share an XCD
    RevWork wk;
    wk.row0 = 64 * tau;
    if (a.rev_kind != kRevChain) {
        const int groups = a.rev_kind == kRevCpAffine ? a.G - 1 : a.G;
        const int bh = u / groups;
        const int gi = u - bh * groups + (a.rev_kind == kRevCpAffine ? 1 : 0);
        const int b = bh / a.H;
        wk.h = bh - b * a.H;
        const int t_begin = gi * a.cpg * kChunk;
        wk.tok0 = (int64_t)b * a.T + t_begin;
        wk.len = min(a.T, (gi + 1) * a.cpg * kChunk) - t_begin;
        wk.su = bh;
        wk.slot0 = (int64_t)bh * a.NC + (int64_t)gi * a.cpg;
        if (a.rev_kind == kRevCpAffine) {
            wk.gin = nullptr;
            wk.gout = a.ws_C + (((int64_t)bh * a.G + gi) * DV + wk.row0) * DK;
            wk.store = false;
        } else {
            wk.gin = gi == a.G - 1 ? (a.dS_final ? a.dS_final + ((int64_t)bh * DV + wk.row0) * DK : nullptr)
                                   : a.ws_E + (((int64_t)bh * a.G + gi) * DV + wk.row0) * DK;
            wk.gout = gi == 0 && a.dS0 ? a.dS0 + ((int64_t)bh * DV + wk.row0) * DK : nullptr;
            wk.store = true;
        }
        return wk;
    }
    const int rank = u / a.H;
    wk.h = u - rank * a.H;
    wk.store = true;
    if (a.cu_seqlens) {
        const int n = a.seq_order ? a.seq_order[rank] : rank;
        wk.tok0 = a.cu_seqlens[n];
        wk.len = a.cu_seqlens[n + 1] - a.cu_seqlens[n];
        wk.su = (int64_t)n * a.H + wk.h;
        wk.slot0 = (int64_t)a.chunk_base[n] * a.H + (int64_t)wk.h * ((wk.len + kChunk - 1) / kChunk);
    } else {
        wk.tok0 = (int64_t)rank * a.T;
        wk.len = a.T;
        wk.su = u;
        wk.slot0 = (int64_t)u * a.NC;
    }
    wk.gin = a.dS_final ? a.dS_final + (wk.su * DV + wk.row0) * DK : nullptr;
    wk.gout = a.dS0 ? a.dS0 + (wk.su * DV + wk.row0) * DK : nullptr;
    return wk;
}

// Chunk of step j (clamped into the sequence: loads past either end re-read
// a valid chunk whose ring slot is never consumed).
__device__ inline int rev_chunk(int NC, int j) { return min(max(NC - 1 - j, 0), NC - 1); }

// T^T of a chunk (64 x 64 bf16 row-major in the workspace) by the 64 lanes of
// wave 4: lane l owns the 16-byte piece l % 8 of rows l / 8 + 8 p.
struct TStager {
    const __bf16 *tg; // T^T of chunk 0 of this unit
    int lane;
    bf16x8 r[2][8];
    __device__ inline void init(const __bf16 *tg_, int lane_) {
        tg = tg_;
        lane = lane_;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int p = 0; p < 8; ++p) r[b][p] = bf16x8{};
    }
    template <int B> __device__ inline void load(int c) {
        const __bf16 *t = tg + (int64_t)c * kChunk * kChunk + (lane / 8) * kChunk + 8 * (lane % 8);
#pragma unroll
        for (int p = 0; p < 8; ++p) r[B][p] = ld8(t + 8 * p * kChunk);
    }
    template <int B> __device__ inline void write(__bf16 *Ts) const {
#pragma unroll
        for (int p = 0; p < 8; ++p) st8(Ts + s64off(lane / 8 + 8 * p, 8 * (lane % 8)), r[B][p]);
    }
};

// The dO tile (64 tokens x this workgroup's 64 values) by the 64 lanes of
// wave 5, as the forward stages V: rows past the end are written as zeros.
struct DStager {
    const __bf16 *dt; // row rv0 of chunk 0, value column col
    int64_t sv;
    int len, rv0, col;
    bf16x8 r[2][8];
    int n[2];
    __device__ inline void init(const __bf16 *dg, int64_t sv_, int len_, int lane) {
        sv = sv_;
        len = len_;
        rv0 = lane / 8;
        col = 8 * (lane % 8);
        dt = dg + rv0 * sv + col;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            n[b] = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) r[b][p] = bf16x8{};
        }
    }
    template <int B> __device__ inline void load(int c) {
        n[B] = rows_of(len, c);
        const __bf16 *b = dt + (int64_t)c * kChunk * sv;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int row = min(rv0 + 8 * p, n[B] - 1);
            r[B][p] = *reinterpret_cast<const bf16x8 *>(b + (int64_t)(row - rv0) * sv);
        }
    }
    template <int B> __device__ inline void write(__bf16 *Ds) const {
        const bf16x8 z = {};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int row = rv0 + 8 * p;
            st8(Ds + s64off(row, col), row < n[B] ? r[B][p] : z);
        }
    }
};

// Waves 6-7: P^T of a chunk as A-operand fragments of the consumer's
// dZ = P^T dO products. Fragment (t, s) holds, in lane (g, c), row 16t + c
// of P^T (column 16t + c of P) over the tokens 32s + {4g + e, 16 + 4g + e}
// (the token order of the dO fragments), i.e. the tiles P[16pa + 4g + e][16pc + c]
// for pc = t and pa = 2s, 2s + 1 in its two halves. The fragments are
// (t, s) = (0,0) (0,1) (1,0) (1,1) (2,1) (3,1); blocks above the diagonal
// (half 0 of (1,0) and of (3,1)) are zero and never written.
__device__ constexpr int rev_frag(int t, int s) { return t < 2 ? 2 * t + s : t + 2; }
template <int DK, int B>
__device__ inline void pt_tiles(const RevBufs<DK> &bf, const QStage<DK> &q, int i, int half, int lane, int g, int c16) {
    KRows<DK> k;
    k_rows<DK>(k, bf.K(i), g, c16);
    __bf16 *Pb = bf.P(i) + 8 * lane;
#pragma unroll
    for (int x = 0; x < 5; ++x) {
        const int pa = kPA[half][x], pc = kPC[half][x];
        const int qi = half ? pa - 1 : (pa == 3 ? 1 : 0);
        // acc[e] = q_{16pa+4g+e} . k_{16pc+c} = P[16pa + 4g + e][16pc + c]
        f32x4 acc = dot_tile<DK>(q.f[B][qi], k.f[pc]);
        if (pa == pc) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = (4 * g + e < c16) ? 0.f : acc[e];
        }
        st4(Pb + 512 * rev_frag(pc, pa >> 1) + 4 * (pa & 1), cvt4(acc));
    }
}

// The consumer's products of one step, each with one LDS operand fragment:
//   V  (j):     Y_t += PT_{t,s} DB_s                  6 steps (Y = dZ, from zero)
//   Y  (t, kb): Y_t += K_{t,kb} GB_kb                 4 * DK/32 steps (GB = bf16(dS'))
//   Q  (m, s):  G^T_m += Q^T_{m,s} DB_s               2 * DK/16 steps, split around Z
//   Z  (j):     Z_t += TT_{t,s} YB_s                  6 steps (Z = dY; TT = rows of T^T)
//   K  (m, s):  G^T_m += K^T_{m,s} ZN_s               2 * DK/16 steps (ZN = bf16(-dY))
template <int DK> struct RevSteps {
    static constexpr int NKB = DK / 32, NMT = DK / 16;
    static constexpr int nV = 6, nY = 4 * NKB, nQ = 2 * NMT, nZ = 6, nK = 2 * NMT;
    static constexpr int bY = nV, bQ1 = bY + nY, bZ = bQ1 + nQ / 2, bQ2 = bZ + nZ, bK = bQ2 + nQ - nQ / 2;
    static constexpr int n = bK + nK;
    static constexpr int depth = 8;
    enum { kV, kY, kQ, kZ, kK };
    static constexpr int kind(int i) {
        return i < bY ? kV : i < bQ1 ? kY : i < bZ ? kQ : i < bQ2 ? kZ : i < bK ? kQ : kK;
    }
    static constexpr int idx(int i) {
        return i < bY ? i : i < bQ1 ? i - bY : i < bZ ? i - bQ1 : i < bQ2 ? i - bZ : i < bK ? i - bQ2 + nQ / 2 : i - bK;
    }
    // V / Z step j -> token tile t and 32-token block s (rev_frag(tT(j), tS(j)) == j)
    static constexpr int tT(int j) { return j < 4 ? j / 2 : j - 2; }
    static constexpr int tS(int j) { return j < 4 ? j % 2 : 1; }
};

template <int DK>
__device__ inline bf16x8 rev_fetch(int i, const __bf16 *K, const __bf16 *Q, const __bf16 *T, const __bf16 *P, int lane,
                                   int g, int c16) {
    using RS = RevSteps<DK>;
    const int k = RS::kind(i), j = RS::idx(i);
    if (k == RS::kV) return ld8(P + 512 * j + 8 * lane);
    if (k == RS::kY) return ld8(K + koff<DK>(16 * (j / RS::NKB) + c16, 32 * (j % RS::NKB) + 8 * g));
    if (k == RS::kQ) return k_trfrag<DK>(Q, j / 2, j % 2, g, c16);
    if (k == RS::kZ) {
        // row 16t + c of T^T over the tokens 32s + {4g + e, 16 + 4g + e}
        const int row = 16 * RS::tT(j) + c16, col = 32 * RS::tS(j) + 4 * g;
        return cat8(ld4(T + s64off(row, col)), ld4(T + s64off(row, col + 16)));
    }
    return k_trfrag<DK>(K, j / 2, j % 2, g, c16);
}

template <int DK, int DV>
__device__ void rev_consumer_loop(const BwdArgs &a, const RevWork &wk, const RevBufs<DK> &bf, int NC, int cw, int lane,
                                  int g, int c16) {
    using RS = RevSteps<DK>;
    constexpr int NMT = DK / 16, D = RS::depth;
    const int lrow = 16 * cw + c16;
    f32x4 G[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
        G[m] = wk.gin ? *reinterpret_cast<const f32x4 *>(wk.gin + lrow * DK + dk_of(m, g)) : f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t sv = (int64_t)a.H * DV;
    __bf16 *dvg = reinterpret_cast<__bf16 *>(a.dv) + wk.tok0 * sv + (int64_t)wk.h * DV + wk.row0 + lrow;
    __bf16 *gout = a.G_chunks + (wk.slot0 * DV + wk.row0 + lrow) * DK;
    __syncthreads(); // matches the producers' prologue
    for (int i = -2; i < NC; ++i) {
        if (i >= 0) {
            const int r = NC - 1 - i, nval = min(kChunk, wk.len - r * kChunk);
            // dS' of chunk r (the gradient of the state after it), for the gradient kernel
            if (wk.store) {
#pragma unroll
                for (int m = 0; m < NMT; ++m) st4(gout + (int64_t)r * DV * DK + dk_of(m, g), cvt4(G[m]));
            }
            const __bf16 *Kb = bf.K(i), *Qb = bf.Q(i), *Tb = bf.Tt(i), *Pb = bf.P(i), *Db = bf.D(i);
            // dO fragments over the tokens 32s + {4g + e, 16 + 4g + e}, this lane's value column
            bf16x8 DB[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int row = 32 * s + 4 * g + (c16 >> 2), col = 16 * cw + 4 * (c16 & 3);
                DB[s] = cat8(tr4(Db + s64off(row, col)), tr4(Db + s64off(row + 16, col)));
            }
            bf16x8 buf[D], GB[RS::NKB], YB[2], ZN[2];
            static_for<0, D>([&](auto ic) { buf[ic.value] = rev_fetch<DK>(ic.value, Kb, Qb, Tb, Pb, lane, g, c16); });
            const bool odd = g & 1;
#pragma unroll
            for (int s = 0; s < RS::NKB; ++s) {
                const bf16x4 lo = cvt4(G[2 * s]), hi = cvt4(G[2 * s + 1]);
                GB[s] = odd ? cat8(hi, lo) : cat8(lo, hi);
            }
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 Y[4], Z[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                Y[t] = zero;
                Z[t] = zero;
            }
            fence();
            static_for<0, RS::n>([&](auto ic) {
                constexpr int i2 = decltype(ic)::value;
                const bf16x8 f = buf[i2 % D];
                if constexpr (i2 + D < RS::n) buf[i2 % D] = rev_fetch<DK>(i2 + D, Kb, Qb, Tb, Pb, lane, g, c16);
                if constexpr (i2 == RS::bZ) {
                    YB[0] = cvt8(Y[0], Y[1]);
                    YB[1] = cvt8(Y[2], Y[3]);
                }
                if constexpr (i2 == RS::bK) {
                    ZN[0] = cvt8(-Z[0], -Z[1]);
                    ZN[1] = cvt8(-Z[2], -Z[3]);
                }
                fence();
                constexpr int k = RS::kind(i2), j = RS::idx(i2);
                if constexpr (k == RS::kV) Y[RS::tT(j)] = mfma32(f, DB[RS::tS(j)], Y[RS::tT(j)]);
                if constexpr (k == RS::kY) Y[j / RS::NKB] = mfma32(f, GB[j % RS::NKB], Y[j / RS::NKB]);
                if constexpr (k == RS::kQ) G[j / 2] = mfma32(f, DB[j % 2], G[j / 2]);
                if constexpr (k == RS::kZ) Z[RS::tT(j)] = mfma32(f, YB[RS::tS(j)], Z[RS::tT(j)]);
                if constexpr (k == RS::kK) G[j / 2] = mfma32(f, ZN[j % 2], G[j / 2]);
                fence();
            });
            // dV = dY: Z[t][e] = dY[16t + 4g + e][lrow]
            if (wk.store) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int tok = 16 * t + 4 * g + e;
                        if (tok < nval) dvg[((int64_t)r * kChunk + tok) * sv] = (__bf16)Z[t][e];
                    }
            }
        }
        __syncthreads();
    }
    if (wk.gout) {
#pragma unroll
        for (int m = 0; m < NMT; ++m) *reinterpret_cast<f32x4 *>(wk.gout + lrow * DK + dk_of(m, g)) = G[m];
    }
}

template <int DK, int DV, int ROLE>
__device__ void rev_producer_loop(const BwdArgs &a, const RevWork &wk, const RevBufs<DK> &bf, int NC, int g, int c16) {
    const int lane = 16 * g + c16;
    const int64_t sqk = (int64_t)a.H * DK, sv = (int64_t)a.H * DV;
    KStager<DK> ks;
    QStage<DK> q;
    TStager ts;
    DStager ds;
    if constexpr (ROLE == 0) {
        ts.init(a.T_chunks + wk.slot0 * kChunk * kChunk, lane);
        ts.template load<0>(rev_chunk(NC, 0));
    }
    if constexpr (ROLE == 1) {
        ds.init(reinterpret_cast<const __bf16 *>(a.dO) + wk.tok0 * sv + (int64_t)wk.h * DV + wk.row0, sv, wk.len, lane);
        ds.template load<0>(rev_chunk(NC, 0));
    }
    if constexpr (ROLE >= 2) {
        ks.init(reinterpret_cast<const __bf16 *>(a.k) + wk.tok0 * sqk + (int64_t)wk.h * DK, sqk, wk.len,
                64 * (ROLE - 2) + lane);
        q.init(reinterpret_cast<const __bf16 *>(a.q) + wk.tok0 * sqk + (int64_t)wk.h * DK, sqk, wk.len, ROLE - 2, g,
               c16);
        ks.template load<0>(rev_chunk(NC, 0));
        ks.template load<1>(rev_chunk(NC, 1));
        q.template load<0>(rev_chunk(NC, 0));
    }
    __syncthreads();
    // Iteration i (consumers on step i):
    //   wave 4:    T^T of step i+1 into LDS, loads of step i+3
    //   wave 5:    dO of step i+1 into LDS, loads of step i+3
    //   waves 6-7: K of step i+2 into LDS (loads of step i+4); Q of step i+1
    //              into LDS and P^T of step i+1 (loads of step i+3)
    // Register sets by step parity; staging is unconditional (clamped chunks
    // land in ring slots that are rewritten before they are read).
    auto iteration = [&](int i, auto ipar) {
        constexpr int PK = decltype(ipar)::value, PS = 1 - PK; // sets of steps i+2 (K) and i+1 (the rest)
        if constexpr (ROLE == 0) {
            ts.template write<PS>(bf.Tt(i + 1));
            ts.template load<PS>(rev_chunk(NC, i + 3));
        } else if constexpr (ROLE == 1) {
            ds.template write<PS>(bf.D(i + 1));
            ds.template load<PS>(rev_chunk(NC, i + 3));
        } else {
            ks.template write<PK>(bf.K(i + 2));
            ks.template load<PK>(rev_chunk(NC, i + 4));
            if (i + 1 >= 0 && i + 1 < NC) {
                q.template write<PS>(bf.Q(i + 1), g);
                pt_tiles<DK, PS>(bf, q, i + 1, ROLE - 2, lane, g, c16);
            }
            q.template load<PS>(rev_chunk(NC, i + 3));
        }
        __syncthreads();
    };
    for (int i = -2; i < NC; i += 2) { // i even
        iteration(i, Int<0>{});
        if (i + 1 < NC) iteration(i + 1, Int<1>{});
    }
}

template <int DK, int DV> __global__ __launch_bounds__(kWsThreads) void rev_chain_kernel(const BwdArgs a) {
    using LY = RevLds<DK>;
    static_assert(LY::total <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::total];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const RevWork wk = rev_work<DK, DV>(a);
    const int NC = (wk.len + kChunk - 1) / kChunk;
    const RevBufs<DK> bf{smem};
    if (NC == 0) { // no tokens: the gradient at the start is the one at the end
        if (wave < 4 && wk.gout) {
            const int lrow = 16 * wave + c16;
#pragma unroll
            for (int m = 0; m < DK / 16; ++m) {
                const int off = lrow * DK + dk_of(m, g);
                *reinterpret_cast<f32x4 *>(wk.gout + off) =
                    wk.gin ? *reinterpret_cast<const f32x4 *>(wk.gin + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        return;
    }
    { // P^T: the blocks above the diagonal are never written; zero both rings once
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 *zp = reinterpret_cast<f32x4 *>(smem + LY::oP);
        for (int x = tid; x < (int)(2 * LY::szP / 16); x += kWsThreads) zp[x] = zero;
    }
    __syncthreads();
    if (wave < 4) {
        rev_consumer_loop<DK, DV>(a, wk, bf, NC, wave, lane, g, c16);
    } else if (wave == 4) {
        rev_producer_loop<DK, DV, 0>(a, wk, bf, NC, g, c16);
    } else if (wave == 5) {
        rev_producer_loop<DK, DV, 1>(a, wk, bf, NC, g, c16);
    } else if (wave == 6) {
        rev_producer_loop<DK, DV, 2>(a, wk, bf, NC, g, c16);
    } else {
        rev_producer_loop<DK, DV, 3>(a, wk, bf, NC, g, c16);
    }
}

template <int DK, int DV> hipError_t launch_rev(const BwdArgs &a, hipStream_t s) {
    const int units = a.rev_kind == kRevChain ? a.B * a.H : a.B * a.H * (a.rev_kind == kRevCpAffine ? a.G - 1 : a.G);
    const int grid = units * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((rev_chain_kernel<DK, DV>), dim3(grid), dim3(kWsThreads), 0, s, a);
    return hipGetLastError();
}

template <int DK, int DV, bool WO> hipError_t launch_ws(const ChainArgs &a, hipStream_t s) {
    const int grid = a.n_units * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    if (a.rows == 128) { // context-parallel transitions at dk = dv = 128, with or without decay
        if constexpr (!WO && DK == 128 && DV == 128) {
            if (a.kind != kCpTransition || a.n_tiles != 2) return hipErrorInvalidValue;
            if (a.g)
                hipLaunchKernelGGL((chain_kernel_ws<DK, DV, false, true, 128, 15>), dim3(grid), dim3(960), 0, s, a);
            else
                hipLaunchKernelGGL((chain_kernel_ws<DK, DV, false, false, 128, 15>), dim3(grid), dim3(960), 0, s, a);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (a.rows == 32) { // narrow tiles: forward with output, dense and packed kinds
        if constexpr (WO) {
            if ((a.kind != kDense && a.kind != kVarlen) || a.n_tiles != DV / 32) return hipErrorInvalidValue;
            if (a.g)
                hipLaunchKernelGGL((chain_kernel_ws<DK, DV, true, true, 32, 8>), dim3(grid), dim3(512), 0, s, a);
            else
                hipLaunchKernelGGL((chain_kernel_ws<DK, DV, true, false, 32, 8>), dim3(grid), dim3(512), 0, s, a);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (a.g)
        hipLaunchKernelGGL((chain_kernel_ws<DK, DV, WO, true, 64, 8>), dim3(grid), dim3(512), 0, s, a);
    else if constexpr (WO)
        hipLaunchKernelGGL((chain_kernel_ws<DK, DV, true, false, 64, 12>), dim3(grid), dim3(768), 0, s, a);
    else // the backward's forward pass and the context-parallel transitions at other widths: 8 waves measured faster than 12
        hipLaunchKernelGGL((chain_kernel_ws<DK, DV, false, false, 64, 8>), dim3(grid), dim3(512), 0, s, a);
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

hipError_t launch_bwd_rev(int dk, int dv, const BwdArgs &a, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_rev<128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_rev<128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_rev<64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_rev<64, 64>(a, stream);
    return hipErrorInvalidValue;
}

} // namespace dn
