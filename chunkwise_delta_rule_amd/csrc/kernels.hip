// gfx950 kernels for the DeltaNet chunkwise-parallel forward pass.
//
// One workgroup (4 waves) owns a 64-row tile of one unit's state and walks
// that unit's chunks in order. Per chunk it runs the per-chunk algorithm of
// "Linear Attention, Visualized" (Haoran Zhang), DeltaNet > "Complete
// per-chunk algorithm", with the state transposed ("Context Parallelism for
// DeltaNet", yywangcs, section 2: S is dv x dk):
//   A  Gram G = K K^T and the masked scores P = (Q K^T) lower-inclusive
//   B  diagonal 16x16 blocks of N = (I + diag(beta) L)^-1 by forward
//      substitution, one wave per block ("Solving for U": unit lower
//      triangular, row by row)
//   C  off-diagonal blocks of N by block forward substitution on the matrix
//      cores; T = N diag(beta) solves (I + diag(beta) L) T = diag(beta)
//   D  W = T K (shared, to LDS as -W) and U = T V (per wave, kept in registers)
//   E  the chain: Z = U - W S^T, O = Q S^T + P Z, S <- S + Z^T K
// Rows of S are independent (row j of S, Z, U and O needs only row j and the
// shared K, Q, W), so each wave owns 16 state rows and runs E on its own;
// only A-D are shared through LDS.
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
#include "dn_internal.h"

namespace dn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename E> struct Tr;

// bf16 operands, fp32 accumulation.
template <> struct Tr<__bf16> {
    using F = bf16x4; // k16 fragment
    using V = bf16x8; // 16-byte vector
    static constexpr int kVec = 8;
    static constexpr int kPad = 8; // LDS row padding, elements (16 bytes)
    __device__ static inline f32x4 mma16(f32x4 c, F a, F b) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 mma32(f32x4 c, F a0, F a1, F b0, F b1) {
        const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline F cvt(f32x4 x) {
        F r;
        r[0] = (__bf16)x[0];
        r[1] = (__bf16)x[1];
        r[2] = (__bf16)x[2];
        r[3] = (__bf16)x[3];
        return r;
    }
    __device__ static inline float tof(__bf16 x) { return (float)x; }
    __device__ static inline __bf16 fromf(float x) { return (__bf16)x; }
};

// fp32 operands: four 16x16x4 products per k16 fragment. Product j takes
// value j of every lane group, i.e. k = 4g + j, so the four together cover the
// 16-deep block once.
template <> struct Tr<float> {
    using F = f32x4;
    using V = f32x4;
    static constexpr int kVec = 4;
    static constexpr int kPad = 4;
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
};

// LDS carve-up of the chain kernel (byte offsets). Row strides are padded by
// 16 bytes so that the 16 rows read by one fragment load fall on distinct banks.
template <typename E, int DK> struct Smem {
    static constexpr int LDK = DK + Tr<E>::kPad;     // Ks, Qs, Ws: [C][LDK]
    static constexpr int LDC = kChunk + Tr<E>::kPad; // Kt: [DK][LDC]; Vt: [R][LDC]; Ts, Ps: [C][LDC]
    static constexpr int LDG = kChunk + 4;           // Gs, Ns (fp32): [C][LDG]
    static constexpr size_t oKs = 0;
    static constexpr size_t oQs = oKs + sizeof(E) * kChunk * LDK;
    static constexpr size_t oKt = oQs + sizeof(E) * kChunk * LDK;
    static constexpr size_t oVt = oKt + sizeof(E) * DK * LDC;
    static constexpr size_t oTs = oVt + sizeof(E) * kRows * LDC;
    static constexpr size_t oPs = oTs + sizeof(E) * kChunk * LDC;
    static constexpr size_t oGs = oPs + sizeof(E) * kChunk * LDC;
    // Ws (-W, element type) shares space with Ns (fp32 diagonal inverses): Ns
    // lives from phase B to C, Ws from D to E.
    static constexpr size_t oWs = oGs + sizeof(float) * kChunk * LDG;
    static constexpr size_t szWs = sizeof(E) * kChunk * LDK;
    static constexpr size_t szNs = sizeof(float) * kChunk * LDG;
    static constexpr size_t oBs = oWs + (szWs > szNs ? szWs : szNs);
    static constexpr size_t total = oBs + sizeof(float) * kChunk;
};

template <typename E> __device__ inline typename Tr<E>::F ldf(const E *p) {
    return *reinterpret_cast<const typename Tr<E>::F *>(p);
}
template <typename E> __device__ inline void stf(E *p, typename Tr<E>::F x) {
    *reinterpret_cast<typename Tr<E>::F *>(p) = x;
}

// Block index -> (unit, tile). Groups of 8 units are interleaved so that all
// tiles of one unit get block indices congruent mod 8: the dispatcher deals
// workgroups round-robin over the 8 XCDs, so the tiles of a unit (which read
// the same K and Q chunks) land on one XCD and share its L2.
__device__ inline void map_block(int x, int n_units, int n_tiles, int &u, int &tau) {
    const int per = 8 * n_tiles;
    const int full = n_units >> 3;
    if (x < full * per) {
        const int grp = x / per, r = x - grp * per;
        u = grp * 8 + (r & 7);
        tau = r >> 3;
    } else {
        const int rem = x - full * per;
        u = full * 8 + rem / n_tiles;
        tau = rem - (rem / n_tiles) * n_tiles;
    }
}

// Off-diagonal blocks of column block b of N = (I + A)^-1, A = diag(beta) L:
//   N_ab = -N_aa * sum_{c=b}^{a-1} A_ac N_cb,   a = b+1..3,
// then T_ab = N_ab diag(beta_b). frag[c] holds N_cb as a k16 B fragment.
template <typename E, int b>
__device__ inline void offdiag_column(typename Tr<E>::F nbb, const float *Gs, const float *Ns,
                                      const float *Bs, E *Ts, int g, int c16, int LDG, int LDC) {
    using TR = Tr<E>;
    using F = typename TR::F;
    F frag[4];
    frag[b] = nbb;
    const float beta_col = Bs[16 * b + c16];
#pragma unroll
    for (int a = b + 1; a < 4; ++a) {
        const float beta_row = Bs[16 * a + c16];
        f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = b; c < a; ++c) {
            f32x4 gr = *reinterpret_cast<const f32x4 *>(Gs + (16 * a + c16) * LDG + 16 * c + 4 * g);
            R = TR::mma16(R, TR::cvt(gr * beta_row), frag[c]);
        }
        const f32x4 nr = *reinterpret_cast<const f32x4 *>(Ns + (16 * a + c16) * LDG + 16 * a + 4 * g);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 nab = -TR::mma16(z, TR::cvt(nr), TR::cvt(R));
        frag[a] = TR::cvt(nab);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Ts[(16 * a + 4 * g + i) * LDC + 16 * b + c16] = TR::fromf(nab[i] * beta_col);
    }
}

template <typename E, int DK, int DV, bool WRITE_O>
__global__ __launch_bounds__(kThreads) void chain_kernel(const ChainArgs a) {
    using TR = Tr<E>;
    using F = typename TR::F;
    using V = typename TR::V;
    using SM = Smem<E, DK>;
    constexpr int NMT = DK / 16;                 // 16-wide dk tiles of the state
    constexpr int NKB = DK / 32;                 // 32-deep k blocks over dk
    constexpr int KQV = DK / TR::kVec;           // 16-byte vectors per K/Q row
    constexpr int NKQ = kChunk * KQV / kThreads; // K (and Q) vectors per thread
    constexpr int VV = kRows / TR::kVec;         // vectors per V-tile row
    constexpr int NVV = kChunk * VV / kThreads;  // V vectors per thread
    constexpr int LDK = SM::LDK, LDC = SM::LDC, LDG = SM::LDG;
    static_assert(NKQ * kThreads == kChunk * KQV && NVV * kThreads == kChunk * VV, "tiling");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SM::total];
    E *Ks = reinterpret_cast<E *>(smem + SM::oKs);
    E *Qs = reinterpret_cast<E *>(smem + SM::oQs);
    E *Kt = reinterpret_cast<E *>(smem + SM::oKt);
    E *Vt = reinterpret_cast<E *>(smem + SM::oVt);
    E *Ts = reinterpret_cast<E *>(smem + SM::oTs);
    E *Ps = reinterpret_cast<E *>(smem + SM::oPs);
    float *Gs = reinterpret_cast<float *>(smem + SM::oGs);
    float *Ns = reinterpret_cast<float *>(smem + SM::oWs);
    E *Ws = reinterpret_cast<E *>(smem + SM::oWs);
    float *Bs = reinterpret_cast<float *>(smem + SM::oBs);

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;

    // ---------------- work decode ----------------
    int u, tau;
    map_block(blockIdx.x, a.n_units, a.n_tiles, u, tau);
    const int H = a.H;
    int64_t tok0 = 0;
    int len = 0, h = 0, row0 = tau * kRows;
    const float *Sin = nullptr;
    float *Sout = nullptr;
    bool identity = false, transposed_out = false, has_v = true;
    if (a.kind == kDense) {
        const int b = u / H;
        h = u - b * H;
        tok0 = (int64_t)b * a.T;
        len = a.T;
        if (a.S0) Sin = a.S0 + ((int64_t)u * DV + row0) * DK;
        if (a.S_final) Sout = a.S_final + ((int64_t)u * DV + row0) * DK;
    } else if (a.kind == kVarlen) {
        const int rank = u / H;
        h = u - rank * H;
        const int n = a.seq_order ? a.seq_order[rank] : rank;
        tok0 = a.cu_seqlens[n];
        len = a.cu_seqlens[n + 1] - a.cu_seqlens[n];
        const int64_t su = (int64_t)n * H + h;
        if (a.S0) Sin = a.S0 + (su * DV + row0) * DK;
        if (a.S_final) Sout = a.S_final + (su * DV + row0) * DK;
    } else {
        const int groups = (a.kind == kCpOutput) ? a.G : a.G - 1;
        const int bh = u / groups;
        const int gi = u - bh * groups;
        const int b = bh / H;
        h = bh - b * H;
        const int t_begin = gi * a.chunks_per_group * kChunk;
        const int t_end = min(a.T, (gi + 1) * a.chunks_per_group * kChunk);
        tok0 = (int64_t)b * a.T + t_begin;
        len = t_end - t_begin;
        const int64_t slot = (int64_t)bh * a.G + gi;
        if (a.kind == kCpOutput) {
            if (gi == 0) {
                if (a.S0) Sin = a.S0 + ((int64_t)bh * DV + row0) * DK;
            } else {
                Sin = a.ws_S + (slot * DV + row0) * DK;
            }
            if (gi == a.G - 1 && a.S_final) Sout = a.S_final + ((int64_t)bh * DV + row0) * DK;
        } else if (tau < DV / kRows) {
            Sout = a.ws_Q + (slot * DV + row0) * DK; // Q_g rows, from a zero start
        } else {
            row0 = (tau - DV / kRows) * kRows; // rows of P_g (dk index), from identity
            identity = true;
            has_v = false;
            transposed_out = true;
            Sout = a.ws_P + slot * DK * DK;
        }
    }

    // ---------------- state init ----------------
    // Sacc[m][i] = S[row0 + 16w + c16][16m + 4g + i]
    const int srow = row0 + 16 * w + c16;
    f32x4 Sacc[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
        if (Sin) {
            Sacc[m] = *reinterpret_cast<const f32x4 *>(Sin + (16 * w + c16) * DK + 16 * m + 4 * g);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Sacc[m][i] = (identity && (16 * m + 4 * g + i) == srow) ? 1.f : 0.f;
        }
    }

    const int NC = (len + kChunk - 1) / kChunk;
    const int64_t sqk = (int64_t)H * DK, sv = (int64_t)H * DV;
    const E *qg = reinterpret_cast<const E *>(a.q) + tok0 * sqk + (int64_t)h * DK;
    const E *kg = reinterpret_cast<const E *>(a.k) + tok0 * sqk + (int64_t)h * DK;
    const E *vg = reinterpret_cast<const E *>(a.v) + tok0 * sv + (int64_t)h * DV + row0;
    const E *bg = reinterpret_cast<const E *>(a.beta) + tok0 * H + h;
    E *og = WRITE_O ? reinterpret_cast<E *>(a.o) + tok0 * sv + (int64_t)h * DV + row0 : nullptr;

    // ---------------- chunk staging (global -> registers -> LDS) ----------------
    V rk[NKQ], rq[NKQ], rv[NVV];
    float rb = 0.f;
    auto gload = [&](int c) {
        const int nval = min(kChunk, len - c * kChunk);
        const int64_t base = (int64_t)c * kChunk;
        const V zero = {};
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int vi = p * kThreads + tid, row = vi / KQV, cv = vi - row * KQV;
            if (row < nval) {
                rk[p] = *reinterpret_cast<const V *>(kg + (base + row) * sqk + cv * TR::kVec);
                rq[p] = *reinterpret_cast<const V *>(qg + (base + row) * sqk + cv * TR::kVec);
            } else {
                rk[p] = zero;
                rq[p] = zero;
            }
        }
        if (has_v) {
#pragma unroll
            for (int p = 0; p < NVV; ++p) {
                const int vi = p * kThreads + tid, row = vi / VV, cv = vi - row * VV;
                rv[p] = (row < nval)
                            ? *reinterpret_cast<const V *>(vg + (base + row) * sv + cv * TR::kVec)
                            : zero;
            }
        }
        if (tid < kChunk) rb = (tid < nval) ? TR::tof(bg[(base + tid) * H]) : 0.f;
    };
    auto lstore = [&]() {
#pragma unroll
        for (int p = 0; p < NKQ; ++p) {
            const int vi = p * kThreads + tid, row = vi / KQV, cv = vi - row * KQV;
            *reinterpret_cast<V *>(Ks + row * LDK + cv * TR::kVec) = rk[p];
            *reinterpret_cast<V *>(Qs + row * LDK + cv * TR::kVec) = rq[p];
#pragma unroll
            for (int e = 0; e < TR::kVec; ++e) Kt[(cv * TR::kVec + e) * LDC + row] = rk[p][e];
        }
        if (has_v) {
#pragma unroll
            for (int p = 0; p < NVV; ++p) {
                const int vi = p * kThreads + tid, row = vi / VV, cv = vi - row * VV;
#pragma unroll
                for (int e = 0; e < TR::kVec; ++e) Vt[(cv * TR::kVec + e) * LDC + row] = rv[p][e];
            }
        }
        if (tid < kChunk) Bs[tid] = rb;
    };

    if (NC > 0) gload(0);
    // T and P are lower triangular: their upper blocks are never written, so
    // zero both once.
    for (int i = tid; i < kChunk * LDC; i += kThreads) {
        Ts[i] = TR::fromf(0.f);
        Ps[i] = TR::fromf(0.f);
    }
    if (NC > 0) lstore();
    __syncthreads();

    f32x4 Zacc[4];
    for (int c = 0; c < NC; ++c) {
        const int nval = min(kChunk, len - c * kChunk);
        if (c + 1 < NC) gload(c + 1);

        // ---- A: Gram and masked scores, lower block pairs (ab >= cb) ----
        // Product p = 2*pair + isP; wave w takes p = w, w+4, ... (waves 0,2: G; 1,3: P).
        {
            const int isP = w & 1;
#pragma unroll
            for (int p = w; p < 20; p += 4) {
                const int pair = p >> 1;
                const int ab = pair >= 6 ? 3 : pair >= 3 ? 2 : pair >= 1 ? 1 : 0;
                const int cb = pair - (ab * (ab + 1)) / 2;
                const E *Ar = Ks + (16 * cb + c16) * LDK;
                const E *Br = (isP ? Qs : Ks) + (16 * ab + c16) * LDK;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    acc = TR::mma32(acc, ldf(Ar + 32 * kb + 4 * g), ldf(Ar + 32 * kb + 16 + 4 * g),
                                    ldf(Br + 32 * kb + 4 * g), ldf(Br + 32 * kb + 16 + 4 * g));
                // acc[i] = k_{16cb+4g+i} . x_{16ab+c16}, x = k (Gram) or q (scores)
                const int row = 16 * ab + c16, col = 16 * cb + 4 * g;
                if (!isP) {
                    *reinterpret_cast<f32x4 *>(Gs + row * LDG + col) = acc;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (col + i > row) acc[i] = 0.f;
                    stf(Ps + row * LDC + col, TR::cvt(acc));
                }
            }
        }
        __syncthreads();

        // ---- B: diagonal blocks N_ww = (I + A_ww)^-1, column c16 per lane ----
        F nfrag;
        {
            const int o = 16 * w;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s = fmaf(Gs[(o + i) * LDG + o + j], x[j], s);
                x[i] = (i == c16 ? 1.f : 0.f) - Bs[o + i] * s;
            }
            if (g == 0) {
                const float bc = Bs[o + c16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    Ns[(o + i) * LDG + o + c16] = x[i];
                    Ts[(o + i) * LDC + o + c16] = TR::fromf(x[i] * bc);
                }
            }
            f32x4 xf;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xf[i] = g == 0 ? x[i] : g == 1 ? x[4 + i] : g == 2 ? x[8 + i] : x[12 + i];
            nfrag = TR::cvt(xf);
        }
        __syncthreads();

        // ---- C: off-diagonal blocks of N, column block w ----
        if (w == 0) offdiag_column<E, 0>(nfrag, Gs, Ns, Bs, Ts, g, c16, LDG, LDC);
        else if (w == 1) offdiag_column<E, 1>(nfrag, Gs, Ns, Bs, Ts, g, c16, LDG, LDC);
        else if (w == 2) offdiag_column<E, 2>(nfrag, Gs, Ns, Bs, Ts, g, c16, LDG, LDC);
        __syncthreads();

        // ---- D: -W = -(T K) to LDS (shared), U = T V for this wave's rows ----
#pragma unroll
        for (int mm = 0; mm < NMT / 4; ++mm) {
            const int m = w * (NMT / 4) + mm;
            const E *Ar = Kt + (16 * m + c16) * LDC;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const E *Br = Ts + (16 * n + c16) * LDC;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= n / 2; ++s)
                    acc = TR::mma32(acc, ldf(Ar + 32 * s + 4 * g), ldf(Ar + 32 * s + 16 + 4 * g),
                                    ldf(Br + 32 * s + 4 * g), ldf(Br + 32 * s + 16 + 4 * g));
                // acc[i] = W[16n + c16][16m + 4g + i]
                stf(Ws + (16 * n + c16) * LDK + 16 * m + 4 * g, TR::cvt(-acc));
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (has_v) {
                const E *Ar = Ts + (16 * t + c16) * LDC;
                const E *Br = Vt + (16 * w + c16) * LDC;
#pragma unroll
                for (int s = 0; s <= t / 2; ++s)
                    acc = TR::mma32(acc, ldf(Ar + 32 * s + 4 * g), ldf(Ar + 32 * s + 16 + 4 * g),
                                    ldf(Br + 32 * s + 4 * g), ldf(Br + 32 * s + 16 + 4 * g));
            }
            Zacc[t] = acc; // U[16t + 4g + i][row 16w + c16]
        }
        __syncthreads();

        // ---- E: the chain, per wave ----
        F SB[NMT];
#pragma unroll
        for (int m = 0; m < NMT; ++m) SB[m] = TR::cvt(Sacc[m]);
        F ZB[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const E *Ar = Ws + (16 * t + c16) * LDK;
            f32x4 z = Zacc[t];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                z = TR::mma32(z, ldf(Ar + 32 * kb + 4 * g), ldf(Ar + 32 * kb + 16 + 4 * g),
                              SB[2 * kb], SB[2 * kb + 1]);
            ZB[t] = TR::cvt(z); // Z[16t + 4g + i][row 16w + c16]
        }
        if constexpr (WRITE_O) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const E *Qr = Qs + (16 * t + c16) * LDK;
                const E *Pr = Ps + (16 * t + c16) * LDC;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    acc = TR::mma32(acc, SB[2 * kb], SB[2 * kb + 1], ldf(Qr + 32 * kb + 4 * g),
                                    ldf(Qr + 32 * kb + 16 + 4 * g));
#pragma unroll
                for (int s = 0; s <= t / 2; ++s)
                    acc = TR::mma32(acc, ZB[2 * s], ZB[2 * s + 1], ldf(Pr + 32 * s + 4 * g),
                                    ldf(Pr + 32 * s + 16 + 4 * g));
                // acc[i] = O[token 16t + c16][row 16w + 4g + i]
                const int tok = 16 * t + c16;
                if (tok < nval)
                    stf(og + ((int64_t)c * kChunk + tok) * sv + 16 * w + 4 * g, TR::cvt(acc));
            }
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            const E *Ar = Kt + (16 * m + c16) * LDC;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Sacc[m] = TR::mma32(Sacc[m], ldf(Ar + 32 * s + 4 * g), ldf(Ar + 32 * s + 16 + 4 * g),
                                    ZB[2 * s], ZB[2 * s + 1]);
        }

        if (c + 1 < NC) {
            __syncthreads();
            lstore();
            __syncthreads();
        }
    }

    // ---------------- state out ----------------
    if (Sout) {
        if (!transposed_out) {
#pragma unroll
            for (int m = 0; m < NMT; ++m)
                *reinterpret_cast<f32x4 *>(Sout + (16 * w + c16) * DK + 16 * m + 4 * g) = Sacc[m];
        } else {
#pragma unroll
            for (int m = 0; m < NMT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) Sout[(int64_t)(16 * m + 4 * g + i) * DK + srow] = Sacc[m][i];
        }
    }
}

// Prefix composition of the group maps for one (b, h) and 16 state rows:
//   S_{g+1} = S_g P_g + Q_g,  g = 0..G-2,  S_0 = S0 (or zero);
// writes S_1..S_{G-1} to ws_S. fp32 throughout (fp32 matrix cores). Each
// wave computes DK/64 of the DK/16 output column tiles; the 16 rows of S are
// exchanged through LDS between steps.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void compose_kernel(const ChainArgs a) {
    constexpr int LDS_ = DK + 4;
    constexpr int TPW = DK / 64;
    __shared__ __attribute__((aligned(16))) float Sl[16 * LDS_];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int rb = blockIdx.x % (DV / 16);
    const int bh = blockIdx.x / (DV / 16);
    for (int idx = tid; idx < 16 * DK; idx += kThreads) {
        const int r = idx / DK, col = idx - r * DK;
        Sl[r * LDS_ + col] = a.S0 ? a.S0[((int64_t)bh * DV + 16 * rb + r) * DK + col] : 0.f;
    }
    __syncthreads();
    for (int gi = 0; gi + 1 < a.G; ++gi) {
        const int64_t slot = (int64_t)bh * a.G + gi;
        const float *Pt = a.ws_P + slot * DK * DK;
        const float *Qg = a.ws_Q + (slot * DV + 16 * rb) * DK;
        f32x4 acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int mt = w * TPW + t;
            acc[t] = *reinterpret_cast<const f32x4 *>(Qg + c16 * DK + 16 * mt + 4 * g);
#pragma unroll
            for (int kk = 0; kk < DK / 16; ++kk) {
                const f32x4 pa = *reinterpret_cast<const f32x4 *>(Pt + (16 * mt + c16) * DK + 16 * kk + 4 * g);
                const f32x4 sb = *reinterpret_cast<const f32x4 *>(Sl + c16 * LDS_ + 16 * kk + 4 * g);
                acc[t] = Tr<float>::mma16(acc[t], pa, sb);
            }
        }
        // acc[t][i] = S_{g+1}[row 16rb + c16][16mt + 4g + i]
        __syncthreads();
        float *Sn = a.ws_S + ((slot + 1) * DV + 16 * rb) * DK;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int mt = w * TPW + t;
            *reinterpret_cast<f32x4 *>(Sl + c16 * LDS_ + 16 * mt + 4 * g) = acc[t];
            *reinterpret_cast<f32x4 *>(Sn + c16 * DK + 16 * mt + 4 * g) = acc[t];
        }
        __syncthreads();
    }
}

template <typename E, int DK, int DV, bool WO>
hipError_t launch_one(const ChainArgs &a, hipStream_t s) {
    const int grid = a.n_units * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((chain_kernel<E, DK, DV, WO>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename E, bool WO> hipError_t launch_dims(int dk, int dv, const ChainArgs &a, hipStream_t s) {
    if constexpr (sizeof(E) == 2) {
        if (dk == 128 && dv == 128) return launch_one<E, 128, 128, WO>(a, s);
        if (dk == 128 && dv == 64) return launch_one<E, 128, 64, WO>(a, s);
        if (dk == 64 && dv == 128) return launch_one<E, 64, 128, WO>(a, s);
        if (dk == 64 && dv == 64) return launch_one<E, 64, 64, WO>(a, s);
    } else {
        if (dk == 64 && dv == 128) return launch_one<E, 64, 128, WO>(a, s);
        if (dk == 64 && dv == 64) return launch_one<E, 64, 64, WO>(a, s);
    }
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_chain(int dtype, int dk, int dv, bool write_o, const ChainArgs &a,
                        hipStream_t stream) {
    if (dtype == 1)
        return write_o ? launch_dims<__bf16, true>(dk, dv, a, stream)
                       : launch_dims<__bf16, false>(dk, dv, a, stream);
    return write_o ? launch_dims<float, true>(dk, dv, a, stream)
                   : launch_dims<float, false>(dk, dv, a, stream);
}

hipError_t launch_compose(int dk, int dv, const ChainArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * (dv / 16);
    if (grid <= 0 || a.G < 2) return hipSuccess;
    if (dk == 128 && dv == 128) hipLaunchKernelGGL((compose_kernel<128, 128>), dim3(grid), dim3(kThreads), 0, stream, a);
    else if (dk == 128 && dv == 64) hipLaunchKernelGGL((compose_kernel<128, 64>), dim3(grid), dim3(kThreads), 0, stream, a);
    else if (dk == 64 && dv == 128) hipLaunchKernelGGL((compose_kernel<64, 128>), dim3(grid), dim3(kThreads), 0, stream, a);
    else if (dk == 64 && dv == 64) hipLaunchKernelGGL((compose_kernel<64, 64>), dim3(grid), dim3(kThreads), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace dn
