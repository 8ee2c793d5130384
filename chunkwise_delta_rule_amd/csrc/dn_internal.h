// Internal interface between the C-ABI layer (api.cpp) and the gfx950
// kernels (kernels.hip). Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dn {

constexpr int kChunk = 64;    // tokens per chunk (C)
constexpr int kRows = 64;     // state rows per workgroup tile
constexpr int kThreads = 256; // 4 waves of 64; each wave owns 16 state rows

// How a workgroup finds its (unit, token range, state source/destination).
enum WorkKind : int {
    kDense = 0,        // one unit per (b, h); whole sequence; writes o
    kVarlen = 1,       // one unit per (sequence, h); writes o
    kCpTransition = 2, // one unit per (b, h, group < G-1); writes P_g^T, Q_g
    kCpOutput = 3,     // one unit per (b, h, group); starts from the composed state; writes o
};

struct ChainArgs {
    const void *q, *k, *v, *beta;
    const float *g; // log decay per token, layout of beta; nullptr: no decay (DeltaNet)
    const float *gk; // Kimi Delta Attention: per-channel log decays, layout of k (fp32)
    void *o;
    const float *S0;
    float *S_final;
    float *S_chunks; // dense kind only, or nullptr: the state entering every chunk,
                     // [B*H][chunks][dv][dk] fp32 (kept for the backward pass)
    __bf16 *T_chunks; // with S_chunks (bf16 DeltaNet without output), or nullptr: T^T of
                      // every chunk, [B*H][chunks][64][64] bf16 row-major (backward pass)
    const int32_t *chunk_base; // varlen with S_chunks: chunks before each sequence, [N + 1];
                               // unit (n, h) owns chunk slots chunk_base[n] H + h NC_n + c
    const int32_t *cu_seqlens;
    const int32_t *seq_order;
    // Context-parallel workspace, per (b*H + h) and group g:
    //   ws_P[((bh * G) + g) * dk * dk]  : P_g transposed (row = output column of S)
    //   ws_Q[((bh * G) + g) * dv * dk]  : Q_g, the group's state from a zero start
    //   ws_S[((bh * G) + g) * dv * dk]  : start state of group g (g >= 1)
    float *ws_P, *ws_Q, *ws_S;
    int kind;
    int B;       // sequences (dense / cp) or N (varlen)
    int H;
    int T;       // tokens per sequence (dense / cp)
    int G;       // groups (cp kinds)
    int chunks_per_group;
    int nh;      // substeps per real token (Gated Delta Product; 1 otherwise, gated kernels only)
    int n_units; // units covered by the grid
    int n_tiles; // 64-row state tiles per unit
};

// One decode step: a single token per unit applied to the state in place.
// q, k: [n_units, dk]; v, o: [n_units, dv]; beta, g: [n_units]; S: [n_units, dv, dk].
struct DecodeArgs {
    const void *q, *k, *v, *beta;
    const float *g;  // log decays, or nullptr (no decay)
    const float *gk; // per-channel log decays [n_units][dk] (Kimi Delta Attention), or nullptr
    float *S;
    void *o;
    int n_units;
    int dv;
};

// Kimi Delta Attention chain (bf16, per-channel log decays a.gk): the work
// kinds of the chain kernels (dense, varlen, context-parallel transitions and
// outputs), grid = n_units * n_tiles workgroups of kThreads threads.
hipError_t launch_kda(int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t stream);

// Backward pass (bf16): gradients of q, k, v, beta and S0 for upstream dO and
// dS_final, from the per-chunk states S_chunks of a forward pass.
struct BwdArgs {
    const void *q, *k, *v, *beta, *dO;
    const float *dS_final; // [B*H][dv][dk] or nullptr (zero)
    const float *S_chunks; // [B*H][NC][dv][dk]: the state entering each chunk
    const __bf16 *T_chunks; // [B*H][NC][64][64]: T^T of each chunk (the forward's), row-major
    float *part;           // [n_tiles][max_slots] blocks of per-tile partial sums
    float *dS0;            // [B*H][dv][dk] or nullptr
    void *dq, *dk, *dv, *dbeta;
    const float *g; // Gated DeltaNet: log decays [tokens][H] (layout of beta), or nullptr
    float *dg;      // their gradient (gated only)
    // varlen: B sequences packed along T (cu_seqlens [B + 1], optional order),
    // chunk slots as in ChainArgs::chunk_base; dense: slot of (unit u, chunk c) = u NC + c
    const int32_t *cu_seqlens, *seq_order, *chunk_base;
    int B, H, T, NC, n_tiles;
    // Gated Delta Product: nh substeps per real token; T, k, v, beta, dk, dv,
    // dbeta are over the virtual sequence, q, g, dO, dq, dg per real token (the
    // query on the last substep, the decay on the first); 1 otherwise
    int nh;
    int64_t max_slots; // chunk slots the workspace holds (dense: B H NC); the finishing grid
};
// Chunk slots before each packed sequence: cb[n] = sum_{m < n} ceil(L_m / 64), cb[N] the total.
hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *cb, hipStream_t stream);
// Floats of one partial block: dP, dT (64 x 64 each), dQ, dK (64 x dk each).
constexpr size_t bwd_part_floats(int dk) { return 2 * 64 * 64 + 2 * 64 * (size_t)dk; }
// Gated: per token k . (row-scaled Z dS') and k . (row-scaled dY S), and per
// wave exp(gamma_C) <dS', S>, after those blocks (padded to 256 floats).
constexpr size_t bwd_part_stride(int dk, bool gated) { return bwd_part_floats(dk) + (gated ? 256 : 0); }
hipError_t launch_bwd(int dk, int dv, const BwdArgs &a, hipStream_t stream);
// Fill n floats with value (a kernel, not a memset, so it can sit in a captured graph).
hipError_t launch_fill(float *p, size_t n, float value, hipStream_t stream);

// Enqueue the decode kernel for dtype (0 = fp32, 1 = bf16) and dk (dv is in
// the arguments; dk, dv in {64, 128}). grid = n_units * dv / 64 workgroups.
hipError_t launch_decode(int dtype, int dk, const DecodeArgs &a, hipStream_t stream);

// Enqueue the chunk-chain kernel for dtype (0 = fp32, 1 = bf16) and (dk, dv).
// grid = n_units * n_tiles workgroups of kThreads threads.
hipError_t launch_chain(int dtype, int dk, int dv, bool write_o, const ChainArgs &a,
                        hipStream_t stream);

// The bf16 chain kernel with specialised waves (chain_bf16.hip); same
// contract as launch_chain, 512 threads per workgroup.
hipError_t launch_chain_bf16(int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t stream);

// Enqueue the prefix composition S_{g+1} = S_g P_g + Q_g for g = 0..G-2,
// writing start states of groups 1..G-1 into ws_S.
hipError_t launch_compose(int dk, int dv, const ChainArgs &a, hipStream_t stream);

} // namespace dn
