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
    kCpTransition = 2, // one unit per (b, h, group of the launch's range); writes P_g^T, Q_g
    kCpOutput = 3,     // one unit per (b, h, group of the launch's range); starts from the
                       // group's start state; writes o
};

struct ChainArgs {
    const void *q, *k, *v, *beta;
    const float *g; // log decay per token, layout of beta; nullptr: no decay (DeltaNet)
    const float *gk; // Kimi Delta Attention: per-channel log decays, layout of k (fp32)
    void *o;
    const float *S0;
    float *S_final;
    __bf16 *S_chunks16; // forward without output for the backward pass, or nullptr: the
                        // state entering every chunk, [slot][dv][dk] bf16 (dense: slot
                        // u NC + c; varlen: chunk_base)
    __bf16 *T_chunks; // with S_chunks16, or nullptr: T^T of
                      // every chunk, [B*H][chunks][64][64] bf16 row-major (backward pass)
    const int32_t *chunk_base; // varlen with S_chunks16: chunks before each sequence, [N + 1];
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
    int n_tiles; // state tiles per unit
    int cp_trans_groups; // groups cp_first..cp_first+cp_trans_groups-1 get a transition
                         // (kCpTransition); 0 reads as those up to G - 2 (the forward pass;
                         // the backward's needs all G)
    int cp_first; // first group of a context-parallel launch (transitions, outputs and the
                  // composition start there; the composition then reads the start state of
                  // that group from ws_S); 0 otherwise
    int cp_count; // kCpOutput: groups cp_first..cp_first+cp_count-1; 0 reads as the rest
    int cp_c0;    // chunks of group 0 (the later groups hold chunks_per_group each, the
                  // last one the rest); 0 reads as chunks_per_group
    int cp_lead;  // kCpOutput: every group but the last also writes its end state into the
                  // start-state slot of the next group in ws_S (group 0 run ahead of the
                  // transitions); 0 otherwise
    int rows;    // state rows per tile of the bf16 chain kernel: 64, or 32 (forward with
                 // output, dense and packed kinds, when the 32-row grid fits on the compute
                 // units in one round), or 128 (context-parallel transitions at dk = dv =
                 // 128: one tile for Q_g, one for P_g); 0 reads as 64
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
// dS_final, from the per-chunk states S_chunks16 of a forward pass.
struct BwdArgs {
    const void *q, *k, *v, *beta, *dO;
    const float *dS_final; // [B*H][dv][dk] or nullptr (zero)
    const __bf16 *T_chunks; // [B*H][NC][64][64]: T^T of each chunk (the forward's), row-major
    const __bf16 *S_chunks16; // the state entering each chunk in bf16 [slot][dv][dk]
    __bf16 *G_chunks;         // reverse-chain pipeline: dS' of each chunk (the gradient of the
                              // state after it) in bf16 [slot][dv][dk]
    unsigned char *part;   // gated: [n_tiles][max_slots] blocks of per-tile partial sums
                           // (bwd_part_bytes each)
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
    // Reverse chain over context-parallel groups of cpg chunks (dense DeltaNet):
    //   kRevCpAffine  groups 1..G-1 from a zero gradient at the group's end, writing only
    //                 the gradient at its start, C_g, to ws_C ([B*H*G][dv][dk] fp32)
    //   kRevCpRun     every group from its composed end gradient (ws_E, or dS_final for
    //                 the last group), writing dv and dS' of its chunks (dS0 from group 0)
    int rev_kind, G, cpg;
    const float *ws_P; // P_g^T of the forward transitions, [B*H*G][dk][dk]
    float *ws_C, *ws_E;
};
enum RevKind { kRevChain = 0, kRevCpAffine = 1, kRevCpRun = 2 };
// Composition of the backward group maps for one (b, h) and 16 state rows:
// E_{G-1} = dS_final (or zero), E_{g-1} = E_g P_g^T + C_g for g = G-1..1, into ws_E.
hipError_t launch_compose_bwd(int dk, int dv, const BwdArgs &a, hipStream_t stream);
// Chunk slots before each packed sequence: cb[n] = sum_{m < n} ceil(L_m / 64), cb[N] the total.
hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *cb, hipStream_t stream);
// Elements of the bf16 sums of one partial block: dP, dT (64 x 64 each), dQ,
// dK (64 x dk each), each summed in fp32 over the tile's 64 values and
// rounded once.
constexpr size_t bwd_part_elems(int dk) { return 2 * 64 * 64 + 2 * 64 * (size_t)dk; }
// Bytes of one partial block: those sums, then in fp32 per token
// k . (row-scaled Z dS') and k . (row-scaled dY S), and per wave
// exp(gamma_C) <dS', S> (padded to 256 floats).
constexpr size_t bwd_part_bytes(int dk) { return bwd_part_elems(dk) * 2 + 256 * 4; }
// The gated backward passes (a.g set): the reverse chain with per-value-tile
// partial sums into a.part, then one finishing workgroup per chunk slot.
hipError_t launch_bwd(int dk, int dv, const BwdArgs &a, hipStream_t stream);
// Chunk-parallel gradients of the reverse-chain pipeline (DeltaNet): dq, dk,
// dbeta from a.S_chunks16 and a.G_chunks. grid = a.max_slots workgroups.
hipError_t launch_bwd_grad(int dk, int dv, const BwdArgs &a, hipStream_t stream);
// Fill n floats with value (a kernel, not a memset, so it can sit in a captured graph).
hipError_t launch_fill(float *p, size_t n, float value, hipStream_t stream);

// Enqueue the decode kernel for dtype (0 = fp32, 1 = bf16) and dk (dv is in
// the arguments; dk, dv in {64, 128}). grid = n_units * dv / 64 workgroups.
hipError_t launch_decode(int dtype, int dk, const DecodeArgs &a, hipStream_t stream);

// Enqueue the chunk-chain kernel for dtype (0 = fp32, 1 = bf16) and (dk, dv).
// grid = n_units * n_tiles workgroups of kThreads threads.
hipError_t launch_chain(int dtype, int dk, int dv, bool write_o, const ChainArgs &a,
                        hipStream_t stream);

// Reverse chain of the DeltaNet backward pass (chain_bf16.hip): per (unit, 64
// value rows), walks the chunks backwards carrying dS, writes dS' of every
// chunk (a.G_chunks), dV and dS0. Needs a.T_chunks. grid = units * n_tiles
// workgroups of 512 threads.
hipError_t launch_bwd_rev(int dk, int dv, const BwdArgs &a, hipStream_t stream);

// The bf16 chain kernel with specialised waves (chain_bf16.hip); same
// contract as launch_chain, 512 threads per workgroup.
hipError_t launch_chain_bf16(int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t stream);

// The dense forward behind deltanet_fwd, deltanet_gated_fwd (g != nullptr)
// and deltanet_gdp_fwd (nh > 1; T counts virtual steps): argument checks,
// group resolution and the launches, with the caller's workspace. Returns a
// DN_* status of include/deltanet.h.
int fwd_dense(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
              void *o, float *S_final, int B, int H, int T, int nh, int dk, int dv, int chunk, int dtype,
              int cp_groups, void *workspace, size_t workspace_bytes, hipStream_t stream, bool allow_side);

// Enqueue the prefix composition S_{g+1} = S_g P_g + Q_g for g = f..G-2,
// f = cp_first (S_0 = S0, or the start state of group f in ws_S when f > 0),
// writing the start states of groups f+1..G-1 into ws_S.
hipError_t launch_compose(int dk, int dv, const ChainArgs &a, hipStream_t stream);

} // namespace dn
