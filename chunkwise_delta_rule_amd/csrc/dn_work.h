// Device-side work decoding shared by the chain kernels: which unit, token
// range, 64-row state tile and state source/destination a workgroup owns.
#pragma once

#include "dn_internal.h"

namespace dn {

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

// What one workgroup works on: a token range of one (sequence, head), a
// 64-row tile of the state, where the tile starts from and where it ends.
struct Work {
    int64_t tok0;
    int len, h, row0;
    int unit;         // index of the (sequence, head) unit
    __bf16 *Schunks16; // rows of the state entering chunk 0 of this unit in bf16 (backward pass), or nullptr
    const float *Sin; // initial rows, or nullptr (zero / identity)
    float *Sout;      // final rows, or nullptr
    bool identity, transposed_out, has_v;
    __bf16 *Tchunks;  // T^T of chunk 0 of this unit (dense kind, first tile only), or nullptr
};

// ROWS: state rows per workgroup tile (64; 32 for the narrow forward tiles,
// dense and packed kinds only; 128 for context-parallel transitions at
// dk = dv = 128).
template <int DK, int DV, int ROWS = kRows> __device__ inline Work decode_work(const ChainArgs &a) {
    int u, tau;
    map_block(blockIdx.x, a.n_units, a.n_tiles, u, tau);
    const int H = a.H;
    Work wk = {0, 0, 0, tau * ROWS, u, nullptr, nullptr, nullptr, false, false, true, nullptr};
    if (a.kind == kDense) {
        const int b = u / H;
        wk.h = u - b * H;
        wk.tok0 = (int64_t)b * a.T;
        wk.len = a.T;
        if (a.S_chunks16)
            wk.Schunks16 = a.S_chunks16 + ((int64_t)u * ((a.T + kChunk - 1) / kChunk) * DV + wk.row0) * DK;
        if (a.T_chunks && tau == 0)
            wk.Tchunks = a.T_chunks + (int64_t)u * ((a.T + kChunk - 1) / kChunk) * kChunk * kChunk;
        if (a.S0) wk.Sin = a.S0 + ((int64_t)u * DV + wk.row0) * DK;
        if (a.S_final) wk.Sout = a.S_final + ((int64_t)u * DV + wk.row0) * DK;
    } else if (a.kind == kVarlen) {
        const int rank = u / H;
        wk.h = u - rank * H;
        const int n = a.seq_order ? a.seq_order[rank] : rank;
        wk.tok0 = a.cu_seqlens[n];
        wk.len = a.cu_seqlens[n + 1] - a.cu_seqlens[n];
        const int64_t su = (int64_t)n * H + wk.h;
        if (a.S0) wk.Sin = a.S0 + (su * DV + wk.row0) * DK;
        if (a.S_final) wk.Sout = a.S_final + (su * DV + wk.row0) * DK;
        if (a.S_chunks16) { // the chunk slots of this unit, contiguous
            const int64_t slot0 = (int64_t)a.chunk_base[n] * H + (int64_t)wk.h * ((wk.len + kChunk - 1) / kChunk);
            wk.Schunks16 = a.S_chunks16 + (slot0 * DV + wk.row0) * DK;
            if (a.T_chunks && tau == 0) wk.Tchunks = a.T_chunks + slot0 * kChunk * kChunk;
        }
    } else {
        const int groups = a.kind == kCpOutput ? (a.cp_count > 0 ? a.cp_count : a.G - a.cp_first)
                                               : (a.cp_trans_groups > 0 ? a.cp_trans_groups : a.G - 1 - a.cp_first);
        const int bh = u / groups;
        const int gi = u - bh * groups + a.cp_first;
        const int b = bh / H;
        wk.h = bh - b * H;
        // first chunk of group i: group 0 holds cp_c0 chunks (0: chunks_per_group),
        // every later group chunks_per_group (the last one the rest)
        const int c0 = a.cp_c0 > 0 ? a.cp_c0 : a.chunks_per_group;
        const int gc0 = gi == 0 ? 0 : c0 + (gi - 1) * a.chunks_per_group;
        const int t_begin = gc0 * kChunk;
        const int t_end = min(a.T, (gi == 0 ? c0 : gc0 + a.chunks_per_group) * kChunk);
        wk.tok0 = (int64_t)b * a.T + t_begin;
        wk.len = t_end - t_begin;
        const int64_t slot = (int64_t)bh * a.G + gi;
        if (a.kind == kCpOutput) {
            if (gi == 0) {
                if (a.S0) wk.Sin = a.S0 + ((int64_t)bh * DV + wk.row0) * DK;
            } else {
                wk.Sin = a.ws_S + (slot * DV + wk.row0) * DK;
            }
            if (gi == a.G - 1) {
                if (a.S_final) wk.Sout = a.S_final + ((int64_t)bh * DV + wk.row0) * DK;
            } else if (a.cp_lead) {
                wk.Sout = a.ws_S + ((slot + 1) * DV + wk.row0) * DK; // the next group's start
            }
            if (a.S_chunks16) { // the backward's forward pass: the group's chunk slots of unit bh
                const int64_t slot0 = (int64_t)bh * ((a.T + kChunk - 1) / kChunk) + gc0;
                wk.Schunks16 = a.S_chunks16 + (slot0 * DV + wk.row0) * DK;
                if (a.T_chunks && tau == 0) wk.Tchunks = a.T_chunks + slot0 * kChunk * kChunk;
            }
        } else if (tau < DV / ROWS) {
            wk.Sout = a.ws_Q + (slot * DV + wk.row0) * DK; // Q_g rows, from a zero start
        } else {
            wk.row0 = (tau - DV / ROWS) * ROWS; // rows of P_g (dk index), from identity
            wk.identity = true;
            wk.has_v = false;
            wk.transposed_out = true;
            wk.Sout = a.ws_P + slot * DK * DK;
        }
    }
    return wk;
}

// Gated Delta Product runs as Gated DeltaNet over a virtual sequence of nh
// substeps per real token ("Linear Attention, Visualized", "GDP as GDN over a
// virtual sequence"): virtual step M is substep M % nh of real token M / nh.
// Queries and outputs live at the real tokens (used on the last substep),
// the decay at the real token (applied on the first substep); keys, values
// and beta are stored per substep, i.e. already in virtual order.
// A work item splits its first virtual step once (64-bit) and then locates
// step first + x with a 32-bit division (x < 2^31 within one sequence).
struct Substep {
    int64_t t;
    int j;
};
struct SubstepBase {
    int64_t t0;  // real token of the first virtual step
    uint32_t j0; // its substep
    uint32_t nh;
};
__device__ inline SubstepBase substep_base(int64_t first, int nh) {
    if (nh == 1) return {first, 0u, 1u};
    const int64_t t = first / nh;
    return {t, (uint32_t)(first - t * nh), (uint32_t)nh};
}
__device__ inline Substep substep_at(const SubstepBase &b, uint32_t x) {
    if (b.nh == 1) return {b.t0 + x, 0};
    const uint32_t y = b.j0 + x, d = y / b.nh;
    return {b.t0 + d, (int)(y - d * b.nh)};
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l gets the sum of
// lanes 0..l): a scan inside each 16-lane row with DPP row shifts (lanes
// shifted in from outside the row read 0), then the totals of the rows below
// added from lanes 15, 31 and 47. Every lane of the wave must be active.
__device__ inline float wave_inclusive_sum(float x, int lane) {
    const int zero = 0;
#define DN_ROW_SHR(N)                                                                                          \
    x += __builtin_bit_cast(                                                                                   \
        float, __builtin_amdgcn_update_dpp(zero, __builtin_bit_cast(int, x), 0x110 + (N), 0xF, 0xF, false))
    DN_ROW_SHR(1);
    DN_ROW_SHR(2);
    DN_ROW_SHR(4);
    DN_ROW_SHR(8);
#undef DN_ROW_SHR
    const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
    const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
    const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
    const int row = lane >> 4;
    return x + (row == 0 ? 0.f : row == 1 ? t0 : row == 2 ? t0 + t1 : t0 + t1 + t2);
}

} // namespace dn
