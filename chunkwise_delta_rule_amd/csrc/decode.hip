// gfx950 kernel for one decode step of DeltaNet / Gated DeltaNet: a single
// token per (sequence, head) applied to a state kept in HBM.
//
// The token recurrence of "Linear Attention, Visualized" (Haoran Zhang),
// DeltaNet > "Recurrent form", "Gated DeltaNet (GDN)" and "Kimi Delta
// Attention (KDA)", with the state S (dv x dk, fp32) acting on column vectors:
//   S <- S D (I - beta k k^T) + beta v k^T,   o = S q
// with D = a I (a = exp(g); a = 1 ungated) or, for KDA, D = Diag(exp(g_j))
// over the key channels j. Per state row r, with w = S[r] D (the decayed row):
//   h_k = w . k,  h_q = w . q,  u = beta (v_r - h_k),
//   S[r] <- w + u k,  o_r = h_q + u (k . q)
// so each row of S is read once and written once, in place.
//
// This is a streaming kernel: 2 dv dk 4 bytes of state per (sequence, head)
// against O(dk + dv) bytes of token data, so HBM bandwidth bounds it and the
// matrix cores have nothing to do. Layout of the work: four lanes per state
// row, each holding dk/4 columns in groups of four; in load step j the four
// lanes of row r read its 64 contiguous bytes 64 j .. 64 j + 63, so every
// load and store instruction moves whole 64-byte segments. The three dot
// products are finished inside each lane quad with two DPP exchanges.
#include "dn_internal.h"

namespace dn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256; // 64 state rows per workgroup

template <typename E> __device__ inline f32x4 load4(const E *p);
template <> __device__ inline f32x4 load4<float>(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
template <> __device__ inline f32x4 load4<__bf16>(const __bf16 *p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// Sum over the four lanes of a quad, returned in all four (DPP quad_perm).
__device__ inline float quad_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)); // [1,0,3,2]
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)); // [2,3,0,1]
    return x;
}

// MODE 0: no decay, 1: scalar decay per unit, 2: per-channel decay (KDA).
template <typename E, int DK, int MODE>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecodeArgs a) {
    constexpr int NJ = DK / 16; // column groups of 4 per lane
    const int tiles = a.dv / 64;
    const int u = blockIdx.x / tiles, tile = blockIdx.x - u * tiles;
    const int p = threadIdx.x & 3, row = 64 * tile + (threadIdx.x >> 2);
    const E *q = reinterpret_cast<const E *>(a.q) + (int64_t)u * DK;
    const E *k = reinterpret_cast<const E *>(a.k) + (int64_t)u * DK;
    const float beta = (float)reinterpret_cast<const E *>(a.beta)[u];
    const float v = (float)reinterpret_cast<const E *>(a.v)[(int64_t)u * a.dv + row];
    const float decay = MODE == 1 ? expf(a.g[u]) : 1.f;
    float *Srow = a.S + ((int64_t)u * a.dv + row) * DK + 4 * p;

    f32x4 s[NJ], kv[NJ];
    float hk = 0.f, hq = 0.f, kq = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) s[j] = *reinterpret_cast<const f32x4 *>(Srow + 16 * j);
    if constexpr (MODE == 2) { // the decayed row w = S[r] Diag(exp(g)) replaces S[r] below
        const float *gk = a.gk + (int64_t)u * DK;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const f32x4 gv = *reinterpret_cast<const f32x4 *>(gk + 16 * j + 4 * p);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[j][e] *= __builtin_amdgcn_exp2f(gv[e] * 1.44269504088896340736f);
        }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        kv[j] = load4<E>(k + 16 * j + 4 * p);
        const f32x4 qv = load4<E>(q + 16 * j + 4 * p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hk = fmaf(s[j][e], kv[j][e], hk);
            hq = fmaf(s[j][e], qv[e], hq);
            kq = fmaf(kv[j][e], qv[e], kq);
        }
    }
    hk = quad_sum(hk);
    hq = quad_sum(hq);
    kq = quad_sum(kq);
    const float corr = beta * (v - decay * hk);
#pragma unroll
    for (int j = 0; j < NJ; ++j) *reinterpret_cast<f32x4 *>(Srow + 16 * j) = decay * s[j] + corr * kv[j];
    if (p == 0) {
        const float o = decay * hq + corr * kq;
        E *op = reinterpret_cast<E *>(a.o) + (int64_t)u * a.dv + row;
        *op = (E)o;
    }
}

template <typename E, int DK> hipError_t launch_dec(const DecodeArgs &a, hipStream_t s) {
    const int grid = a.n_units * (a.dv / 64);
    if (grid <= 0) return hipSuccess;
    if (a.gk)
        hipLaunchKernelGGL((decode_kernel<E, DK, 2>), dim3(grid), dim3(kDecThreads), 0, s, a);
    else if (a.g)
        hipLaunchKernelGGL((decode_kernel<E, DK, 1>), dim3(grid), dim3(kDecThreads), 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<E, DK, 0>), dim3(grid), dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_decode(int dtype, int dk, const DecodeArgs &a, hipStream_t stream) {
    if (dtype == 1) return dk == 128 ? launch_dec<__bf16, 128>(a, stream) : launch_dec<__bf16, 64>(a, stream);
    return dk == 128 ? launch_dec<float, 128>(a, stream) : launch_dec<float, 64>(a, stream);
}

} // namespace dn
