// Chunk-parallel gradients of the DeltaNet backward pass (gfx950, bf16).
//
// The forward per chunk ("Linear Attention, Visualized", DeltaNet > "Complete
// per-chunk algorithm", with S transposed as in "Context Parallelism for
// DeltaNet", section 2) is
//   L = strict-lower(K K^T),  N = (I + diag(beta) L)^-1,  T = N diag(beta)
//   P = lower-inclusive(Q K^T),  Y = V - K S^T,  Z = T Y
//   O = Q S^T + P Z,  S' = S + Z^T K.
// The pages give no backward pass; this is its reverse mode. Given the state
// S entering a chunk (stored by the forward pass) and dS' (the gradient of
// the state after it, stored by the reverse chain), every other gradient of
// the chunk is local:
//   dZ = P^T dO + K dS'^T,   dY = T^T dZ
//   dP = lower-inclusive(dO Z^T),   dT = lower-inclusive(dZ Y^T)
//   dQ = dO S + dP K
//   dK = dP^T Q + Z dS' - dY S + (dL + dL^T) K
//   X = N^T dT,  dbeta_t = X_tt + sum_j dA_tj (K K^T)_tj
//   dA = strict-lower(-(X diag(beta)) N^T),  dL = diag(beta) dA
// with N^T = I - L^T T^T (from N (I + diag(beta) L) = I). dV = dY and dS0
// come from the reverse chain, which forms the same dY.
//
// One workgroup (4 waves) per chunk slot. The value dimension is walked in
// quarters of 32 values, so that the LDS of a workgroup stays under 80 KB and
// two workgroups share a CU. Per quarter:
//   A1  wave w = (value tile vt = w % 2, token pair tg = w / 2) forms Y and
//       dZ for token tiles 2 tg, 2 tg + 1 of its 16 values; both go to LDS;
//   A2  the same wave forms Z = T Y and dY = T^T dZ for those tiles, taking
//       the other pair's Y or dZ tiles from LDS;
//   B   wave w accumulates, for token rows 16 w .. 16 w + 15, the quarter's
//       share of dP, dT, dO S and Z dS' - dY S in registers;
// the next quarter's S, dS', V and dO are loaded from HBM during the current
// one. The finishing products (Gram matrix, N^T, X, dA) then run on the
// 64 x 64 chunk matrices.
//
// Matrix-core layout (16x16x32 and 16x16x16 bf16, wave64, lane l = 16 g + c):
// an operand lane supplies row (or column) c and the contraction slots of its
// group g; the accumulator's lane holds D[4 g + i][c]. Contractions over dk
// give group g the 8 consecutive slots 8 g .. 8 g + 7, so K, Q, S and dS'
// rows are single 16-byte reads. Contractions over tokens or values give
// group g the slots 4 g + e and 16 + 4 g + e of each 32-block, read either as
// 8-byte row pieces or by the transposing read ds_read_b64_tr_b16 (a provider
// lane supplies 4 consecutive columns of one row, receivers get one column
// over 4 rows). Every 16x16 tile that one wave produces for others is stored
// transposed, so that its accumulator layout becomes one 8-byte write per
// lane (D^T[col][4 g .. 4 g + 3]); its readers swap row and column reads.
//
// LDS layouts: rows padded and a few row bits XORed into the low bits of the
// column unit, so that the accesses above are free of bank conflicts (64 banks
// for reads: 16 lanes per pass for 16-byte reads, 32 for 8-byte and
// transposing ones; 32 banks for writes: 8 lanes per pass for 16-byte writes,
// 16 for 8-byte ones) while an address stays affine in the 16-row and
// 16-column block indices, so that one register plus immediate offsets
// serves a loop over blocks:
//   o64   64-column tiles (T^T, the Y/Z/dZ/dY^T quarter tiles, dP^T, dT^T,
//         L^T and dL^T, N, (X diag(beta))^T): rows of 80, 8-byte units,
//         row bit 2 -> unit bit 0, row bit 3 -> unit bit 1;
//   o64p  P: rows of 72, row bit 3 -> unit bit 0 (two-way conflicts on the
//         transposing reads, which only the first phase makes);
//   okk   dk-column tiles (K, Q, S, dS'): rows of dk + 16, 16-byte units,
//         row bit 3 -> unit bit 0;
//   ov    32-column quarter tiles of dO: unpadded 16-byte units, row bit 2 ->
//         unit bit 1, row bit 3 -> unit bit 0.
// V enters only as the starting value of the Y accumulators and is read from
// HBM straight into their layout.
#include "dn_internal.h"

namespace dn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kGT = 256; // threads per workgroup

__device__ inline f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
// Round to nearest even, two packed conversions reassembled through words.
__device__ inline bf16x4 cvt4(f32x4 x) {
    const bf16x2 lo = __builtin_convertvector(__builtin_shufflevector(x, x, 0, 1), bf16x2);
    const bf16x2 hi = __builtin_convertvector(__builtin_shufflevector(x, x, 2, 3), bf16x2);
    const u32x2 u = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    return __builtin_bit_cast(bf16x4, u);
}
__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ inline bf16x8 neg8(bf16x8 x) { // sign flip, exact
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    const unsigned m = 0x80008000u;
    return __builtin_bit_cast(bf16x8, u32x4{u[0] ^ m, u[1] ^ m, u[2] ^ m, u[3] ^ m});
}
__device__ inline bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x4 ld4(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ inline void st4(__bf16 *p, bf16x4 x) { *reinterpret_cast<bf16x4 *>(p) = x; }
__device__ inline void st8(__bf16 *p, bf16x8 x) { *reinterpret_cast<bf16x8 *>(p) = x; }
// Transposing read: this lane supplies the 8 bytes at p (4 consecutive
// columns of one row) and receives its column over the 4 supplied rows.
__device__ inline bf16x4 tr4(const __bf16 *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
}

// Element offsets of the LDS layouts (see the file header).
__device__ inline int o64(int r, int c) { // 64 columns, rows of 80
    return r * 80 + 4 * ((c >> 2) ^ (((r >> 2) & 1) | (((r >> 3) & 1) << 1))) + (c & 3);
}
__device__ inline int o64p(int r, int c) { // 64 columns, rows of 72 (P)
    return r * 72 + 4 * ((c >> 2) ^ ((r >> 3) & 1)) + (c & 3);
}
template <int DK> __device__ inline int okk(int r, int c) {
    return r * (DK + 16) + 8 * ((c >> 3) ^ ((r >> 3) & 1)) + (c & 7);
}
__device__ inline int ov(int r, int c) {
    const int s = (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
    return r * 32 + 8 * ((c >> 3) ^ s) + (c & 7);
}
// Per-lane element offsets of the access patterns, for the blocks at (0, 0);
// a block 16 x rows and 16 y columns away adds 16 x times the row length
// plus 16 y (every layout above keeps that affine), so one register and
// immediate offsets serve a loop over blocks.
struct Offs {
    int g, c;
    int t64, r64;     // o64: transposing-read provider (4 g + c / 4, 4 (c % 4)); 8-byte piece (c, 4 g)
    int t64p, r64p;   // o64p: the same
    int tkk, r8kk;    // okk: transposing-read provider; 16-byte piece (c, 8 g)
    int tv, rv0, rv1; // ov: provider (4 g + c / 4, 16 vt + 4 (c % 4)); pieces (c, 4 g), (c, 16 + 4 g)
};
// Formed from an opaque copy of the lane index: each phase forms its own
// offsets where it uses them, instead of the compiler keeping (or spilling)
// the offsets of every phase live from the first one.
template <int DK> __device__ inline Offs offs(int lane, int vt) {
    int l = lane;
    asm volatile("" : "+v"(l));
    Offs o;
    o.g = l >> 4;
    o.c = l & 15;
    const int tr = 4 * o.g + (o.c >> 2), tc = 4 * (o.c & 3);
    o.t64 = o64(tr, tc);
    o.r64 = o64(o.c, 4 * o.g);
    o.t64p = o64p(tr, tc);
    o.r64p = o64p(o.c, 4 * o.g);
    o.tkk = okk<DK>(tr, tc);
    o.r8kk = okk<DK>(o.c, 8 * o.g);
    o.tv = ov(tr, 16 * vt + tc);
    o.rv0 = ov(o.c, 4 * o.g);
    o.rv1 = ov(o.c, 16 + 4 * o.g);
    return o;
}

template <int DK> struct GradLds {
    static constexpr size_t szK = (size_t)64 * (DK + 16) * 2; // K (Q at the start and at the end)
    static constexpr size_t szQt = (size_t)32 * (DK + 16) * 2; // a quarter of S or dS'
    static constexpr size_t sz64 = 64 * 80 * 2, sz32 = 32 * 80 * 2, szP = 64 * 72 * 2, szD = 64 * 32 * 2;
    static constexpr size_t oK = 0, oTT = oK + szK, oB = oTT + sz64, oDa = oB + 256, oR = oDa + 256;
    // quarter phase: P, S, dS', dO, Y^T, Z^T, dZ^T, dY^T (Q over the last four at the start)
    static constexpr size_t oP = oR, oS = oP + szP, oG = oS + szQt, oD = oG + szQt;
    static constexpr size_t oY = oD + szD, oZ = oY + sz32, odZ = oZ + sz32, odY = odZ + sz32, end = odY + sz32;
    // finish: dP^T, L^T (then dL^T), dT^T, N, (X diag(beta))^T (Q over dT^T and N at the end)
    static constexpr size_t fdP = oR, fL = fdP + sz64, fdT = fL + sz64, fN = fdT + sz64, fX = fN + sz64;
    static constexpr size_t fend = fX + sz64;
    static constexpr size_t total = end > fend ? end : fend;
    static_assert(4 * sz32 >= szK && 2 * sz64 >= szK, "Q fits over the tiles it shares");
};

// Two waves per SIMD (two workgroups per CU): at most 256 registers per lane.
template <int DK, int DV>
__global__ __launch_bounds__(kGT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_grad_kernel(const BwdArgs a) {
    using E = __bf16;
    using LY = GradLds<DK>;
    constexpr int NKB = DK / 32, NMT = DK / 16, NQ = DV / 32;
    constexpr int KU = DK / 8;              // 16-byte units per dk row
    constexpr int NKV = 64 * KU / kGT;      // K (and Q) units per thread
    constexpr int NSV = 32 * KU / kGT;      // units of a quarter of S (and dS') per thread
    constexpr int RK = DK + 16;             // row length of the dk-column tiles
    static_assert(LY::total <= 80 * 1024, "two workgroups per CU");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::total];
    E *Ks = reinterpret_cast<E *>(smem + LY::oK), *TT = reinterpret_cast<E *>(smem + LY::oTT);
    float *Bt = reinterpret_cast<float *>(smem + LY::oB), *dba = reinterpret_cast<float *>(smem + LY::oDa);
    E *Ps = reinterpret_cast<E *>(smem + LY::oP), *Ss = reinterpret_cast<E *>(smem + LY::oS);
    E *Gs = reinterpret_cast<E *>(smem + LY::oG);
    E *Ds = reinterpret_cast<E *>(smem + LY::oD), *YT = reinterpret_cast<E *>(smem + LY::oY);
    E *ZT = reinterpret_cast<E *>(smem + LY::oZ), *dZT = reinterpret_cast<E *>(smem + LY::odZ);
    E *dYT = reinterpret_cast<E *>(smem + LY::odY);
    E *Q0 = YT; // Q while P is formed
    E *dPT = reinterpret_cast<E *>(smem + LY::fdP), *dTT = reinterpret_cast<E *>(smem + LY::fdT);
    E *LT = reinterpret_cast<E *>(smem + LY::fL), *Ns = reinterpret_cast<E *>(smem + LY::fN);
    E *XT = reinterpret_cast<E *>(smem + LY::fX);
    E *Q1 = dTT; // Q for the last products (over dT^T and N)

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    int g = lane >> 4, c = lane & 15;
    // chunk slot s = blockIdx.x -> sequence, head h and chunk r
    const int64_t s = blockIdx.x;
    int64_t tok0;
    int len, h, r;
    if (a.cu_seqlens) {
        // slots of sequence n: [cb[n] H, cb[n + 1] H), head-major; the grid covers
        // the workspace's slot bound, so trailing workgroups return at once
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
    const int64_t sqk = (int64_t)a.H * DK, sv = (int64_t)a.H * DV, t0 = tok0 + (int64_t)r * kChunk;
    const int nval = min(kChunk, len - r * kChunk); // >= 1: slots exist only for chunks with tokens
    const E *kg = reinterpret_cast<const E *>(a.k) + t0 * sqk + (int64_t)h * DK;
    const E *qg = reinterpret_cast<const E *>(a.q) + t0 * sqk + (int64_t)h * DK;
    const E *vg = reinterpret_cast<const E *>(a.v) + t0 * sv + (int64_t)h * DV;
    const E *dg = reinterpret_cast<const E *>(a.dO) + t0 * sv + (int64_t)h * DV;
    const E *Sg = a.S_chunks16 + s * DV * DK, *Gg = a.G_chunks + s * DV * DK;
    const E *Tg = a.T_chunks + s * kChunk * kChunk;

    // ---- HBM loads: K, Q, T^T, beta, the first quarter ----
    bf16x8 kv[NKV], qv[NKV];
    bf16x4 tv[4];
#pragma unroll
    for (int p = 0; p < NKV; ++p) {
        const int vi = p * kGT + tid, row = vi / KU, u = vi % KU;
        const uint32_t off = (uint32_t)(min(row, nval - 1) * sqk + 8 * u);
        kv[p] = ld8(kg + off);
        qv[p] = ld8(qg + off);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) tv[p] = ld4(Tg + (uint32_t)(4 * (p * kGT + tid)));
    const float bt = (w == 0 && lane < nval) ? (float)reinterpret_cast<const E *>(a.beta)[(t0 + lane) * a.H + h] : 0.f;
    // per quarter: S, dS' and dO for LDS, and the V entries this lane's Y tiles
    // start from (token 16 (2 tg + j) + 4 g + i, value 16 vt + c of the quarter),
    // rows past the chunk's end masked to zero when used
    const int vt = w & 1, tg = w >> 1;
    bf16x8 sq[NSV], gq[NSV], dq;
    E vy[2][4], vcur[2][4];
    auto load_quarter = [&](int tau) {
#pragma unroll
        for (int p = 0; p < NSV; ++p) {
            const int vi = p * kGT + tid, row = vi / KU, u = vi % KU;
            const uint32_t off = (uint32_t)((32 * tau + row) * DK + 8 * u);
            sq[p] = ld8(Sg + off);
            gq[p] = ld8(Gg + off);
        }
        const uint32_t off = (uint32_t)(min(tid >> 2, nval - 1) * sv + 32 * tau + 8 * (tid & 3));
        dq = ld8(dg + off);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (2 * tg + j) + 4 * (lane >> 4) + i;
                vy[j][i] = vg[(uint32_t)(min(row, nval - 1) * sv + 32 * tau + 16 * vt + (lane & 15))];
            }
    };
    auto stage_quarter = [&]() {
#pragma unroll
        for (int p = 0; p < NSV; ++p) {
            const int vi = p * kGT + tid, row = vi / KU, u = vi % KU;
            st8(Ss + okk<DK>(row, 8 * u), sq[p]);
            st8(Gs + okk<DK>(row, 8 * u), gq[p]);
        }
        const int row = tid >> 2, u = tid & 3;
        st8(Ds + ov(row, 8 * u), row < nval ? dq : bf16x8{});
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) vcur[j][i] = vy[j][i];
    };
    load_quarter(0);
#pragma unroll
    for (int p = 0; p < NKV; ++p) { // rows past the chunk's end are zero
        const int vi = p * kGT + tid, row = vi / KU, u = vi % KU;
        const bool on = row < nval;
        st8(Ks + okk<DK>(row, 8 * u), on ? kv[p] : bf16x8{});
        st8(Q0 + okk<DK>(row, 8 * u), on ? qv[p] : bf16x8{});
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int vi = p * kGT + tid;
        st4(TT + o64(vi >> 4, 4 * (vi & 15)), tv[p]);
    }
    if (w == 0) Bt[lane] = bt;
    stage_quarter();
    __syncthreads();
    if (NQ > 1) load_quarter(1);

    Offs o = offs<DK>(lane, vt);
    g = o.g;
    c = o.c;
    // ---- P = lower-inclusive(Q K^T): the ten 16 x 16 tiles (a, b <= a) ----
    {
        const int nt = w < 2 ? 3 : 2;
#pragma unroll
        for (int it = 0; it < 3; ++it) {
            if (it >= nt) break;
            // wave 0: (0,0) (3,0) (3,1); 1: (1,0) (1,1) (3,2); 2: (2,0) (2,1); 3: (2,2) (3,3)
            const int code = w == 0 ? (it == 0 ? 0x00 : it == 1 ? 0x30 : 0x31)
                           : w == 1 ? (it == 0 ? 0x10 : it == 1 ? 0x11 : 0x32)
                           : w == 2 ? (it == 0 ? 0x20 : 0x21)
                                    : (it == 0 ? 0x22 : 0x33);
            const int ta = code >> 4, tb = code & 15;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                acc = mfma32(ld8(Ks + o.r8kk + RK * 16 * tb + 32 * kb), ld8(Q0 + o.r8kk + RK * 16 * ta + 32 * kb),
                             acc);
            // acc[e] = k_{16 tb + 4 g + e} . q_{16 ta + c} = P[16 ta + c][16 tb + 4 g + e]
            const int row = 16 * ta + c, col = 16 * tb + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = col + e > row ? 0.f : acc[e];
            st4(Ps + o.r64p + 72 * 16 * ta + 16 * tb, cvt4(acc));
        }
    }
    __syncthreads(); // P complete; Q's tiles free for Y^T ..

    // sums over the value dimension for token rows 16 w + 4 g + i: dP and dT
    // tiles (w, s2), dO S and Z dS' - dY S (dk columns 16 m + c)
    f32x4 pp[4], tt[4], dQa[NMT], dKa[NMT];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        pp[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
        tt[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
        dQa[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        dKa[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tau = 0; tau < NQ; ++tau) {
        if (tau > 0) {
            stage_quarter();
            __syncthreads();
            if (tau + 1 < NQ) load_quarter(tau + 1);
        }
        o = offs<DK>(lane, vt);
        g = o.g;
        c = o.c;
        // A1: Y = V - K S^T and dZ = P^T dO + K dS'^T for token tiles 2 tg, 2 tg + 1
        // and the 16 values 16 vt + c of the quarter
        bf16x4 yb[2], zb[2];
        {
            bf16x8 sr[NKB], gr[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sr[kb] = neg8(ld8(Ss + o.r8kk + RK * 16 * vt + 32 * kb));
                gr[kb] = ld8(Gs + o.r8kk + RK * 16 * vt + 32 * kb);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = 2 * tg + j;
                f32x4 ay;
#pragma unroll
                for (int i = 0; i < 4; ++i) ay[i] = 16 * t + 4 * g + i < nval ? (float)vcur[j][i] : 0.f;
                f32x4 zk = {0.f, 0.f, 0.f, 0.f}, zp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 kr = ld8(Ks + o.r8kk + RK * 16 * t + 32 * kb);
                    ay = mfma32(kr, sr[kb], ay);
                    zk = mfma32(kr, gr[kb], zk);
                }
                // the two product shapes accumulate separately and are added after
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    if (s2 >= t)
                        zp = mfma16(tr4(Ps + o.t64p + 72 * 16 * s2 + 16 * t),
                                    tr4(Ds + o.tv + 32 * 16 * s2), zp);
                yb[j] = cvt4(ay);
                zb[j] = cvt4(zp + zk);
                st4(YT + o.r64 + 80 * 16 * vt + 16 * t, yb[j]);
                st4(dZT + o.r64 + 80 * 16 * vt + 16 * t, zb[j]);
            }
        }
        __syncthreads();
        o = offs<DK>(lane, vt);
        g = o.g;
        c = o.c;
        // A2: Z = T Y and dY = T^T dZ for the same tiles
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = 2 * tg + j;
            f32x4 z = {0.f, 0.f, 0.f, 0.f}, dy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                if (s2 <= t) {
                    const bf16x4 yf = (s2 >> 1) == tg ? yb[s2 & 1] : ld4(YT + o.r64 + 80 * 16 * vt + 16 * s2);
                    z = mfma16(tr4(TT + o.t64 + 80 * (16 * s2) + 16 * t), yf, z);
                }
                if (s2 >= t) {
                    const bf16x4 zf = (s2 >> 1) == tg ? zb[s2 & 1] : ld4(dZT + o.r64 + 80 * 16 * vt + 16 * s2);
                    dy = mfma16(ld4(TT + o.r64 + 80 * 16 * t + 16 * s2), zf, dy);
                }
            }
            st4(ZT + o.r64 + 80 * 16 * vt + 16 * t, cvt4(z));
            st4(dYT + o.r64 + 80 * 16 * vt + 16 * t, cvt4(dy));
        }
        __syncthreads();
        o = offs<DK>(lane, vt);
        g = o.g;
        c = o.c;
        // B: the quarter's share of the sums, token rows 16 w .. 16 w + 15
        {
            const bf16x8 aO = cat8(ld4(Ds + o.rv0 + 32 * 16 * w), ld4(Ds + o.rv1 + 32 * 16 * w));
            const bf16x8 aZ = cat8(tr4(ZT + o.t64 + 80 * (0) + 16 * w),
                                   tr4(ZT + o.t64 + 80 * (16) + 16 * w));
            const bf16x8 adZ = cat8(tr4(dZT + o.t64 + 80 * (0) + 16 * w),
                                    tr4(dZT + o.t64 + 80 * (16) + 16 * w));
            const bf16x8 adYn = neg8(cat8(tr4(dYT + o.t64 + 80 * (0) + 16 * w),
                                          tr4(dYT + o.t64 + 80 * (16) + 16 * w)));
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                if (s2 > w) break; // dP and dT are lower-inclusive
                const bf16x8 bZ = cat8(tr4(ZT + o.t64 + 80 * (0) + 16 * s2),
                                       tr4(ZT + o.t64 + 80 * (16) + 16 * s2));
                const bf16x8 bY = cat8(tr4(YT + o.t64 + 80 * (0) + 16 * s2),
                                       tr4(YT + o.t64 + 80 * (16) + 16 * s2));
                pp[s2] = mfma32(aO, bZ, pp[s2]);
                tt[s2] = mfma32(adZ, bY, tt[s2]);
            }
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                const bf16x8 bS = cat8(tr4(Ss + o.tkk + RK * (0) + 16 * m),
                                       tr4(Ss + o.tkk + RK * (16) + 16 * m));
                const bf16x8 bG = cat8(tr4(Gs + o.tkk + RK * (0) + 16 * m),
                                       tr4(Gs + o.tkk + RK * (16) + 16 * m));
                dQa[m] = mfma32(aO, bS, dQa[m]);
                dKa[m] = mfma32(aZ, bG, dKa[m]);
                dKa[m] = mfma32(adYn, bS, dKa[m]);
            }
        }
        __syncthreads(); // the quarter's tiles are no longer read
    }

    // ---- finish ----
    o = offs<DK>(lane, vt);
    g = o.g;
    c = o.c;
    // dP^T and dT^T (lower-inclusive), and L^T from this wave's Gram rows
    // gm[j][i] = k_t . k_{16 j + c}, t = 16 w + 4 g + i
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        f32x4 x = pp[s2], y = tt[s2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool on = 16 * s2 + c <= 16 * w + 4 * g + i;
            x[i] = on ? x[i] : 0.f;
            y[i] = on ? y[i] : 0.f;
        }
        st4(dPT + o.r64 + 80 * 16 * s2 + 16 * w, cvt4(x));
        st4(dTT + o.r64 + 80 * 16 * s2 + 16 * w, cvt4(y));
    }
    f32x4 gm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gm[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            gm[j] = mfma32(ld8(Ks + o.r8kk + RK * 16 * w + 32 * kb), ld8(Ks + o.r8kk + RK * 16 * j + 32 * kb),
                           gm[j]);
        f32x4 l = gm[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) l[i] = 16 * j + c < 16 * w + 4 * g + i ? l[i] : 0.f;
        st4(LT + o.r64 + 80 * 16 * j + 16 * w, cvt4(l));
    }
    __syncthreads();
    o = offs<DK>(lane, vt);
    g = o.g;
    c = o.c;
    // N^T = I - L^T T^T, row block w (upper triangular: blocks b >= w), stored as N
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (b >= w) {
#pragma unroll
            for (int k0 = 0; k0 < 64; k0 += 32)
                acc = mfma32(cat8(ld4(LT + o.r64 + 80 * 16 * w + k0), ld4(LT + o.r64 + 80 * 16 * w + k0 + 16)),
                             cat8(tr4(TT + o.t64 + 80 * (k0) + 16 * b),
                                  tr4(TT + o.t64 + 80 * (k0 + 16) + 16 * b)),
                             acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = (16 * w + 4 * g + i == 16 * b + c ? 1.f : 0.f) - acc[i];
        st4(Ns + o.r64 + 80 * 16 * b + 16 * w, cvt4(acc));
    }
    __syncthreads();
    o = offs<DK>(lane, vt);
    g = o.g;
    c = o.c;
    // X = N^T dT: dbeta_a = diag X; (X diag(beta))^T to LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += 32)
            x = mfma32(cat8(tr4(Ns + o.t64 + 80 * (k0) + 16 * w),
                            tr4(Ns + o.t64 + 80 * (k0 + 16) + 16 * w)),
                       cat8(ld4(dTT + o.r64 + 80 * 16 * j + k0), ld4(dTT + o.r64 + 80 * 16 * j + k0 + 16)), x);
        const float bc = Bt[16 * j + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (j == w && c == 4 * g + i) dba[16 * w + 4 * g + i] = x[i];
        st4(XT + o.r64 + 80 * 16 * j + 16 * w, cvt4(x * bc));
    }
    __syncthreads();
    o = offs<DK>(lane, vt);
    g = o.g;
    c = o.c;
    // dA = strict-lower(-(X diag(beta)) N^T); dbeta_b = sum_j dA_tj gm_tj; dL = diag(beta) dA,
    // stored as dL^T over L^T
    float dbb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += 32)
            da = mfma32(cat8(tr4(XT + o.t64 + 80 * (k0) + 16 * w),
                             tr4(XT + o.t64 + 80 * (k0 + 16) + 16 * w)),
                        cat8(ld4(Ns + o.r64 + 80 * 16 * j + k0), ld4(Ns + o.r64 + 80 * 16 * j + k0 + 16)), da);
        f32x4 dl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * w + 4 * g + i;
            const float dai = 16 * j + c < t ? -da[i] : 0.f;
            dbb[i] += dai * gm[j][i];
            dl[i] = Bt[t] * dai;
        }
        st4(LT + o.r64 + 80 * 16 * j + 16 * w, cvt4(dl));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) // sum over the 16 lanes of the row group
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) dbb[i] += __shfl_xor(dbb[i], o, 16);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NKV; ++p) { // N and (X diag(beta))^T are no longer read: Q goes over them
        const int vi = p * kGT + tid, row = vi / KU, u = vi % KU;
        st8(Q1 + okk<DK>(row, 8 * u), row < nval ? qv[p] : bf16x8{});
    }
    __syncthreads();
    o = offs<DK>(lane, vt);
    g = o.g;
    c = o.c;
    // dQ += dP K;  dK += dP^T Q + dL K + dL^T K
    bf16x8 aPc[2], aPr[2], aLc[2], aLr[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int k0 = 32 * h2;
        aPc[h2] = cat8(tr4(dPT + o.t64 + 80 * (k0) + 16 * w),
                       tr4(dPT + o.t64 + 80 * (k0 + 16) + 16 * w));
        aPr[h2] = cat8(ld4(dPT + o.r64 + 80 * 16 * w + k0), ld4(dPT + o.r64 + 80 * 16 * w + k0 + 16));
        aLc[h2] = cat8(tr4(LT + o.t64 + 80 * (k0) + 16 * w),
                       tr4(LT + o.t64 + 80 * (k0 + 16) + 16 * w));
        aLr[h2] = cat8(ld4(LT + o.r64 + 80 * 16 * w + k0), ld4(LT + o.r64 + 80 * 16 * w + k0 + 16));
    }
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int k0 = 32 * h2;
            const bf16x8 kc = cat8(tr4(Ks + o.tkk + RK * (k0) + 16 * m),
                                   tr4(Ks + o.tkk + RK * (k0 + 16) + 16 * m));
            const bf16x8 qc = cat8(tr4(Q1 + o.tkk + RK * (k0) + 16 * m),
                                   tr4(Q1 + o.tkk + RK * (k0 + 16) + 16 * m));
            dQa[m] = mfma32(aPc[h2], kc, dQa[m]);
            dKa[m] = mfma32(aPr[h2], qc, dKa[m]);
            dKa[m] = mfma32(aLc[h2], kc, dKa[m]);
            dKa[m] = mfma32(aLr[h2], kc, dKa[m]);
        }
    E *dkg = reinterpret_cast<E *>(a.dk) + t0 * sqk + (int64_t)h * DK;
    E *dqg = reinterpret_cast<E *>(a.dq) + t0 * sqk + (int64_t)h * DK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * g + i;
        if (t < nval) {
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                dqg[(int64_t)t * sqk + 16 * m + c] = (E)dQa[m][i];
                dkg[(int64_t)t * sqk + 16 * m + c] = (E)dKa[m][i];
            }
            if (c == 0) reinterpret_cast<E *>(a.dbeta)[(t0 + t) * a.H + h] = (E)(dba[t] + dbb[i]);
        }
    }
}

template <int DK, int DV> hipError_t launch_grad(const BwdArgs &a, hipStream_t s) {
    if (a.max_slots <= 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_grad_kernel<DK, DV>), dim3((unsigned)a.max_slots), dim3(kGT), 0, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_bwd_grad(int dk, int dv, const BwdArgs &a, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_grad<128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_grad<128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_grad<64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_grad<64, 64>(a, stream);
    return hipErrorInvalidValue;
}

} // namespace dn
