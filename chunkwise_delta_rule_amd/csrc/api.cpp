// C-ABI of the DeltaNet forward library: argument checks, context-parallel
// planning and dispatch to the gfx950 kernels. Every check runs before the
// first launch, so an error return means nothing was enqueued.
#include "../../include/deltanet.h"
#include "dn_internal.h"

#include <mutex>
#include <stdint.h>

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int check_shape(int dk, int dv, int chunk, int dtype) {
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_ERR_INVALID;
    if (dk <= 0 || dv <= 0 || chunk <= 0) return DN_ERR_INVALID;
    if (chunk != dn::kChunk) return DN_ERR_UNSUPPORTED;
    if (dtype == DN_BF16) {
        if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return DN_ERR_UNSUPPORTED;
    } else {
        if (dk != 64 || (dv != 64 && dv != 128)) return DN_ERR_UNSUPPORTED;
    }
    return DN_OK;
}

// Compute units of the current device, cached per device ordinal.
int device_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Choice of group count for cp_groups = 0. The serial pass keeps one
// workgroup per (unit, 64-row tile) busy for the whole chunk chain. When
// those workgroups fill at least half of the compute units, splitting only
// adds the transition work. Otherwise the chain is cut into enough groups to
// give every compute unit an output workgroup, keeping at least 8 chunks per
// group so the per-group transition cost stays amortised. With `lead` (the
// forward at dk = dv = 128, whose group 0 runs its output chain beside the
// transitions of the others), groups 1..G-1 take the compute units in the
// output phase, so there is one group more.
int pick_groups(int B, int H, int T, int dv, bool lead) {
    const int nc = (T + dn::kChunk - 1) / dn::kChunk;
    const int serial_wgs = B * H * (dv / dn::kRows);
    const int cus = device_cus();
    if (serial_wgs * 2 >= cus || nc < 16) return 1;
    int G = cus / serial_wgs;
    if (lead && G >= 2) G += 1;
    if (G > nc / 8) G = nc / 8;
    return G < 1 ? 1 : G;
}

// Whether the dense forward runs group 0 ahead (see fwd_dense): the shapes
// whose transitions take one 128-row tile each for Q_g and P_g, so that the
// transitions of groups 1..G-2 and the output chain of group 0 together
// occupy as many workgroups as the output phase of groups 1..G-1.
bool fwd_lead_shape(int dk, int dv) { return dk == 128 && dv == 128; }

// State rows per workgroup tile of the bf16 forward with output on the
// serial chain: 32 when the 32-row grid still fits on the compute units in
// one round (twice the workgroups of the 64-row grid, each with half the
// consumer work and its producer work spread over six waves, so a chunk takes
// about a fifth less time), else 64 (a second round would cost more).
int pick_rows(int dtype, int n_units, int dv) {
    if (dtype != DN_BF16) return dn::kRows;
    return (int64_t)n_units * (dv / 32) <= device_cus() ? 32 : dn::kRows;
}

// Resolve the requested group count into (G, chunks per group) with no empty group.
void resolve_groups(int requested, int B, int H, int T, int dv, int &G, int &cpg, bool lead = false) {
    const int nc = (T + dn::kChunk - 1) / dn::kChunk;
    G = requested == 0 ? pick_groups(B, H, T, dv, lead) : requested;
    if (G > nc) G = nc;
    if (G < 1) G = 1;
    cpg = nc > 0 ? (nc + G - 1) / G : 1;
    G = nc > 0 ? (nc + cpg - 1) / cpg : 1;
}

size_t ws_bytes_for(int B, int H, int dk, int dv, int G) {
    if (G <= 1) return 0;
    return (size_t)B * H * G * ((size_t)dk * dk + 2 * (size_t)dv * dk) * sizeof(float);
}

// A second stream per device for work that runs beside the caller's stream
// inside one call, ordered by a fork event recorded on the caller's stream
// and a join event the caller's stream waits for. Created on first use (at
// the default priority) and kept until the process ends.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool failed = false;
};
constexpr int kMaxSideDevices = 64;
std::mutex side_mu; // guards the table and every fork/join sequence (the events are shared)
SideStream side_table[kMaxSideDevices];

// The current device's side stream, or nullptr (creation failed, or the
// caller's stream is being captured: then nothing is created or forked and
// the work runs on the caller's stream). Called with side_mu held.
SideStream *side_stream(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
    SideStream &e = side_table[dev];
    if (e.failed) return nullptr;
    if (!e.s) {
        if (hipStreamCreateWithFlags(&e.s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&e.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&e.join, hipEventDisableTiming) != hipSuccess) {
            e.failed = true; // what was created stays; the caller's stream serves from now on
            return nullptr;
        }
    }
    return &e;
}

// Enqueues launch_lead (group 0 ahead) on `stream` and launch_trans (the
// transitions of the other groups) beside it: the transitions go to the
// device's second stream, forked from `stream` by an event (so they follow
// the caller's earlier work) and joined back into it by another (so the
// caller's later work follows them). The second stream's start waits for the
// fork event, a few microseconds, so the longer chain, group 0's, stays on
// `stream`. Without a second stream (allow_side false, creation failed, or
// `stream` being captured) both run one after the other on `stream`.
template <class F0, class F1>
hipError_t launch_beside(hipStream_t stream, bool allow_side, F0 &&launch_lead, F1 &&launch_trans) {
    std::lock_guard<std::mutex> lock(side_mu);
    SideStream *sd = allow_side ? side_stream(stream) : nullptr;
    if (!sd) {
        const hipError_t e = launch_lead(stream);
        return e == hipSuccess ? launch_trans(stream) : e;
    }
    hipError_t e = hipEventRecord(sd->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(sd->s, sd->fork, 0);
    if (e != hipSuccess) return e;
    const hipError_t e1 = launch_trans(sd->s);
    e = hipEventRecord(sd->join, sd->s);
    if (e != hipSuccess) return e;
    const hipError_t e0 = launch_lead(stream);
    e = hipStreamWaitEvent(stream, sd->join, 0);
    return e != hipSuccess ? e : e1 != hipSuccess ? e1 : e0;
}

} // namespace

namespace dn {

// Dense forward, with (g != nullptr) or without the per-token decay. T counts
// virtual steps: nh substeps per real token (Gated Delta Product; nh = 1
// otherwise), so q, g and o hold T / nh real tokens per sequence.
int fwd_dense(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
              void *o, float *S_final, int B, int H, int T, int nh, int dk, int dv, int chunk, int dtype,
              int cp_groups, void *workspace, size_t workspace_bytes, hipStream_t stream, bool allow_side) {
    int st = check_shape(dk, dv, chunk, dtype);
    if (st != DN_OK) return st;
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0) return DN_ERR_INVALID;
    const size_t esz = dtype == DN_BF16 ? 2 : 4;
    if (T > 0) {
        if (!q || !k || !v || !beta || !o) return DN_ERR_INVALID;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return DN_ERR_INVALID;
        if (!aligned_to(beta, esz)) return DN_ERR_INVALID;
        if (g && !aligned_to(g, 4)) return DN_ERR_INVALID;
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return DN_ERR_INVALID;
    if ((int64_t)B * H > (int64_t)1 << 24) return DN_ERR_UNSUPPORTED;

    int G, cpg;
    resolve_groups(cp_groups, B, H, T, dv, G, cpg, fwd_lead_shape(dk, dv));
    const size_t need = ws_bytes_for(B, H, dk, dv, G);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return DN_ERR_WORKSPACE;

    dn::ChainArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.o = o;
    a.S0 = S0;
    a.S_final = S_final;
    a.B = B;
    a.H = H;
    a.T = T;
    a.nh = nh;
    hipError_t err;
    if (G <= 1) {
        a.kind = dn::kDense;
        a.n_units = B * H;
        a.rows = pick_rows(dtype, a.n_units, dv);
        a.n_tiles = dv / a.rows;
        err = dn::launch_chain(dtype, dk, dv, true, a, stream);
        return err == hipSuccess ? DN_OK : DN_ERR_HIP;
    }
    float *ws = static_cast<float *>(workspace);
    const size_t per = (size_t)B * H * G;
    a.ws_P = ws;
    a.ws_Q = a.ws_P + per * dk * dk;
    a.ws_S = a.ws_Q + per * dv * dk;
    a.G = G;
    a.chunks_per_group = cpg;
    // Group 0 starts from S0, which is known: at dk = dv = 128 with three or
    // more groups it runs its output chain (writing the start state of group
    // 1) beside the transitions of groups 1..G-2, on the compute units those
    // leave free, and the output phase covers groups 1..G-1 only.
    const bool lead = dtype == DN_BF16 && fwd_lead_shape(dk, dv) && G >= 3;
    const int first = lead ? 1 : 0;
    if (lead) {
        // Group 0's chain (with output) costs about 5% more per chunk than a
        // transition chain (two 128-row tiles), and the transitions start a
        // few microseconds later; so group 0 takes the remainder of an even
        // split over G - 0.05 groups, about 5% fewer chunks than the others,
        // and both end together. The count of groups stays G.
        const int nc = (T + dn::kChunk - 1) / dn::kChunk;
        const int c = (int)((nc * 20LL + 20LL * G - 2) / (20LL * G - 1)); // ceil(nc / (G - 0.05))
        const int c0 = nc - (G - 1) * c;
        if (c0 >= 1 && c0 <= c) {
            a.chunks_per_group = c;
            a.cp_c0 = c0;
        }
    }
    dn::ChainArgs a0 = a;
    if (lead) {
        a0.kind = dn::kCpOutput;
        a0.cp_first = 0;
        a0.cp_count = 1;
        a0.cp_lead = 1;
        a0.S_final = nullptr;
        a0.rows = dn::kRows;
        a0.n_units = B * H;
        a0.n_tiles = dv / dn::kRows;
    }
    // (i) group transitions for groups first..G-2: at dk = dv = 128, one
    // 128-row tile for Q_g and one for P_g (the chunk's Gram tiles, inverses
    // and T formed once per 128 state rows); else 64-row tiles
    a.kind = dn::kCpTransition;
    a.cp_first = first;
    a.n_units = B * H * (G - 1 - first);
    a.rows = (dtype == DN_BF16 && dk == 128 && dv == 128) ? 128 : dn::kRows;
    a.n_tiles = dv / a.rows + dk / a.rows;
    if (lead) {
        err = launch_beside(
            stream, allow_side, [&](hipStream_t s) { return dn::launch_chain(dtype, dk, dv, true, a0, s); },
            [&](hipStream_t s) { return dn::launch_chain(dtype, dk, dv, false, a, s); });
    } else {
        err = dn::launch_chain(dtype, dk, dv, false, a, stream);
    }
    if (err != hipSuccess) return DN_ERR_HIP;
    // (ii) prefix composition of the maps -> start states of groups first+1..G-1
    err = dn::launch_compose(dk, dv, a, stream);
    if (err != hipSuccess) return DN_ERR_HIP;
    // (iii) every group from first on from its start state, writing o (and
    // S_final from the last group)
    a.kind = dn::kCpOutput;
    a.rows = dn::kRows;
    a.n_units = B * H * (G - first);
    a.n_tiles = dv / dn::kRows;
    err = dn::launch_chain(dtype, dk, dv, true, a, stream);
    return err == hipSuccess ? DN_OK : DN_ERR_HIP;
}

} // namespace dn

namespace {
using dn::fwd_dense;

int fwd_varlen(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
               void *o, float *S_final, const int32_t *cu_seqlens, const int32_t *seq_order, int N, int total_T,
               int H, int dk, int dv, int chunk, int dtype, hipStream_t stream) {
    int st = check_shape(dk, dv, chunk, dtype);
    if (st != DN_OK) return st;
    if (N <= 0 || H <= 0 || total_T < 0 || !cu_seqlens) return DN_ERR_INVALID;
    const size_t esz = dtype == DN_BF16 ? 2 : 4;
    if (total_T > 0) {
        if (!q || !k || !v || !beta || !o) return DN_ERR_INVALID;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return DN_ERR_INVALID;
        if (!aligned_to(beta, esz)) return DN_ERR_INVALID;
        if (g && !aligned_to(g, 4)) return DN_ERR_INVALID;
    }
    if (!aligned_to(cu_seqlens, 4) || (seq_order && !aligned_to(seq_order, 4))) return DN_ERR_INVALID;
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return DN_ERR_INVALID;
    if ((int64_t)N * H > (int64_t)1 << 24) return DN_ERR_UNSUPPORTED;

    dn::ChainArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.o = o;
    a.S0 = S0;
    a.S_final = S_final;
    a.cu_seqlens = cu_seqlens;
    a.seq_order = seq_order;
    a.kind = dn::kVarlen;
    a.nh = 1;
    a.B = N;
    a.H = H;
    a.T = total_T;
    a.n_units = N * H;
    a.rows = pick_rows(dtype, a.n_units, dv);
    a.n_tiles = dv / a.rows;
    hipError_t err = dn::launch_chain(dtype, dk, dv, true, a, stream);
    return err == hipSuccess ? DN_OK : DN_ERR_HIP;
}

} // namespace

namespace {
size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

// Workspace bytes per chunk slot of the backward pass. DeltaNet: the state
// entering the chunk and the gradient of the state leaving it (bf16), then
// T^T of the chunk (bf16). The gated passes: the state entering the chunk
// (bf16) and the per-value-tile partial sums (bf16 sums, fp32 per-token
// extras), then T^T of the chunk (bf16).
size_t bwd_slot_bytes(int dk, int dv, bool gated) {
    const size_t tt = (size_t)dn::kChunk * dn::kChunk * sizeof(__bf16);
    if (!gated) return 2 * (size_t)dv * dk * sizeof(__bf16) + tt;
    return (size_t)dv * dk * sizeof(__bf16) + (size_t)(dv / dn::kRows) * dn::bwd_part_bytes(dk) + tt;
}

// Chunk slots of a packed batch, bounded without reading the lengths:
// sum_n ceil(L_n / 64) <= total_T / 64 + N.
size_t varlen_max_slots(int N, int total_T, int H) {
    return ((size_t)total_T / dn::kChunk + (size_t)N) * (size_t)H;
}

// The backward pass, dense (cu_seqlens NULL: B sequences of T tokens) or
// packed (B = N sequences, T = total tokens). Workspace, DeltaNet: [S entering
// each chunk (bf16) | dS leaving each chunk (bf16) | T^T of each chunk | chunk
// offsets (varlen)]; gated: [S entering each chunk (fp32) | partial sums |
// T^T of each chunk | chunk offsets (varlen)].
int bwd_common(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
               const void *dO, const float *dS_final, void *dq, void *dk_, void *dv_, void *dbeta, float *dg,
               float *dS0, const int32_t *cu_seqlens, const int32_t *seq_order, int B, int H, int T, int nh, int dk,
               int dv, int chunk, int dtype, void *workspace, size_t workspace_bytes, size_t need,
               hipStream_t stream, int cp_groups = 1) {
    int st = check_shape(dk, dv, chunk, dtype);
    if (st != DN_OK) return st;
    if (dtype != DN_BF16) return DN_ERR_UNSUPPORTED;
    if ((int64_t)B * H > (int64_t)1 << 24) return DN_ERR_UNSUPPORTED;
    if (H > 65536) return DN_ERR_UNSUPPORTED; // the gradient kernel's in-chunk offsets stay within 32 bits
    if (T > 0) {
        if (!q || !k || !v || !beta || !dO || !dq || !dk_ || !dv_ || !dbeta) return DN_ERR_INVALID;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned_to(beta, 2) ||
            !aligned_to(dq, 2) || !aligned_to(dk_, 2) || !aligned_to(dv_, 2) || !aligned_to(dbeta, 2))
            return DN_ERR_INVALID;
        if (g && (!dg || !aligned_to(g, 4) || !aligned_to(dg, 4))) return DN_ERR_INVALID;
    }
    if ((S0 && !aligned16(S0)) || (dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0)))
        return DN_ERR_INVALID;
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return DN_ERR_WORKSPACE;
    const bool varlen = cu_seqlens != nullptr;
    const int NC = varlen ? 0 : (T + dn::kChunk - 1) / dn::kChunk;
    if (!varlen && NC == 0) { // no tokens: the gradient of S0 is the gradient of the final state
        if (dS0) {
            const size_t n = (size_t)B * H * dv * dk * sizeof(float);
            const hipError_t e = dS_final ? hipMemcpyAsync(dS0, dS_final, n, hipMemcpyDeviceToDevice, stream)
                                          : dn::launch_fill(dS0, n / sizeof(float), 0.f, stream);
            if (e != hipSuccess) return DN_ERR_HIP;
        }
        return DN_OK;
    }
    const size_t slots = varlen ? varlen_max_slots(B, T, H) : (size_t)B * H * NC;
    if (slots > (size_t)INT32_MAX) return DN_ERR_UNSUPPORTED; // one finishing workgroup per chunk slot
    const bool gated = g != nullptr;
    unsigned char *part = nullptr;
    __bf16 *S16 = nullptr, *G16 = nullptr, *Tck;
    if (gated) {
        S16 = static_cast<__bf16 *>(workspace);
        part = reinterpret_cast<unsigned char *>(S16 + slots * dv * dk);
        Tck = reinterpret_cast<__bf16 *>(part + slots * (dv / dn::kRows) * dn::bwd_part_bytes(dk));
    } else {
        S16 = static_cast<__bf16 *>(workspace);
        G16 = S16 + slots * dv * dk;
        Tck = G16 + slots * dv * dk;
    }
    int32_t *cb = varlen ? reinterpret_cast<int32_t *>(Tck + slots * dn::kChunk * dn::kChunk) : nullptr;
    if (varlen && dn::launch_chunk_base(cu_seqlens, B, cb, stream) != hipSuccess) return DN_ERR_HIP;
    // pass 1: the forward chain, keeping the state entering every chunk and its T
    dn::ChainArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.S0 = S0;
    a.S_chunks16 = S16;
    a.T_chunks = Tck;
    a.chunk_base = cb;
    a.cu_seqlens = cu_seqlens;
    a.seq_order = seq_order;
    a.B = B;
    a.H = H;
    a.T = T;
    a.nh = nh;
    a.kind = varlen ? dn::kVarlen : dn::kDense;
    a.n_units = B * H;
    a.n_tiles = dv / dn::kRows;
    // context parallelism (dense DeltaNet): G groups of cpg chunks
    int G = 1, cpg = NC;
    if (!varlen && cp_groups != 1) resolve_groups(cp_groups, B, H, T, dv, G, cpg);
    float *cws = nullptr;
    if (G > 1) {
        // [P_g^T | Q_g, then C_g | S_g, then E_g] per (b*H + h, g), after the per-chunk slots
        cws = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(workspace) + bwd_slot_bytes(dk, dv, gated) * slots);
        const size_t per = (size_t)B * H * G;
        a.ws_P = cws;
        a.ws_Q = a.ws_P + per * dk * dk;
        a.ws_S = a.ws_Q + per * dv * dk;
        a.G = G;
        a.chunks_per_group = cpg;
        // (i) the transitions of every group (the reverse chain needs P_g of groups 1..G-1)
        a.kind = dn::kCpTransition;
        a.cp_trans_groups = G;
        a.n_units = B * H * G;
        a.rows = (dk == 128 && dv == 128) ? 128 : dn::kRows;
        a.n_tiles = dv / a.rows + dk / a.rows;
        if (dn::launch_chain(dtype, dk, dv, false, a, stream) != hipSuccess) return DN_ERR_HIP;
        a.cp_trans_groups = 0;
        // (ii) the start states of groups 1..G-1
        if (dn::launch_compose(dk, dv, a, stream) != hipSuccess) return DN_ERR_HIP;
        // (iii) every group from its start state, keeping the state entering each chunk and its T
        a.kind = dn::kCpOutput;
        a.n_units = B * H * G;
        a.rows = dn::kRows;
        a.n_tiles = dv / dn::kRows;
    }
    if (dn::launch_chain(dtype, dk, dv, false, a, stream) != hipSuccess) return DN_ERR_HIP;
    // DeltaNet: the reverse chain of the state gradients (with dv and dS0),
    // then every chunk's dq, dk, dbeta in parallel. Gated: the backward chain
    // with per-tile partial sums, then the finishing pass.
    dn::BwdArgs b = {};
    b.q = q;
    b.k = k;
    b.v = v;
    b.beta = beta;
    b.dO = dO;
    b.dS_final = dS_final;
    b.S_chunks16 = S16;
    b.G_chunks = G16;
    b.T_chunks = Tck;
    b.part = part;
    b.dS0 = dS0;
    b.dq = dq;
    b.dk = dk_;
    b.dv = dv_;
    b.dbeta = dbeta;
    b.g = g;
    b.dg = dg;
    b.cu_seqlens = cu_seqlens;
    b.seq_order = seq_order;
    b.chunk_base = cb;
    b.B = B;
    b.H = H;
    b.T = T;
    b.nh = nh;
    b.NC = NC;
    b.n_tiles = dv / dn::kRows;
    b.max_slots = (int64_t)slots;
    if (G > 1) {
        // reverse chain over the groups: C_g of groups 1..G-1 from a zero end gradient,
        // the composed end gradients E_g, then every group from E_g (gated: the
        // backward chain with its partial sums, then the finishing pass)
        const size_t per = (size_t)B * H * G;
        b.G = G;
        b.cpg = cpg;
        b.ws_P = cws;
        b.ws_C = cws + per * dk * dk;
        b.ws_E = b.ws_C + per * dv * dk;
        b.rev_kind = dn::kRevCpAffine;
        if ((gated ? dn::launch_bwd(dk, dv, b, stream) : dn::launch_bwd_rev(dk, dv, b, stream)) != hipSuccess)
            return DN_ERR_HIP;
        if (dn::launch_compose_bwd(dk, dv, b, stream) != hipSuccess) return DN_ERR_HIP;
        b.rev_kind = dn::kRevCpRun;
        if ((gated ? dn::launch_bwd(dk, dv, b, stream) : dn::launch_bwd_rev(dk, dv, b, stream)) != hipSuccess)
            return DN_ERR_HIP;
        b.rev_kind = dn::kRevChain;
        if (!gated && dn::launch_bwd_grad(dk, dv, b, stream) != hipSuccess) return DN_ERR_HIP;
    } else if (gated) {
        if (dn::launch_bwd(dk, dv, b, stream) != hipSuccess) return DN_ERR_HIP;
    } else {
        if (dn::launch_bwd_rev(dk, dv, b, stream) != hipSuccess) return DN_ERR_HIP;
        if (dn::launch_bwd_grad(dk, dv, b, stream) != hipSuccess) return DN_ERR_HIP;
    }
    return DN_OK;
}
} // namespace

namespace {
// One decode step for every (sequence, head): g is a scalar log decay per
// unit (Gated DeltaNet), gk a per-channel one (Kimi Delta Attention); at most
// one of them is given.
int decode_common(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *gk,
                  float *S, void *o, int B, int H, int dk, int dv, int dtype, hipStream_t stream) {
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_ERR_INVALID;
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0) return DN_ERR_INVALID;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return DN_ERR_UNSUPPORTED;
    if ((int64_t)B * H > (int64_t)1 << 24) return DN_ERR_UNSUPPORTED;
    const size_t esz = dtype == DN_BF16 ? 2 : 4;
    if (!q || !k || !v || !beta || !S || !o) return DN_ERR_INVALID;
    if (!aligned_to(q, 4 * esz) || !aligned_to(k, 4 * esz) || !aligned_to(v, esz) || !aligned_to(beta, esz) ||
        !aligned_to(o, esz) || !aligned16(S) || (g && !aligned_to(g, 4)) || (gk && !aligned16(gk)))
        return DN_ERR_INVALID;
    dn::DecodeArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.g = g;
    a.gk = gk;
    a.S = S;
    a.o = o;
    a.n_units = B * H;
    a.dv = dv;
    return dn::launch_decode(dtype, dk, a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}
} // namespace

extern "C" {

const char *deltanet_status_string(int status) {
    switch (status) {
    case DN_OK: return "ok";
    case DN_ERR_INVALID: return "invalid argument";
    case DN_ERR_UNSUPPORTED: return "unsupported shape or chunk size";
    case DN_ERR_WORKSPACE: return "workspace missing or too small";
    case DN_ERR_HIP: return "HIP runtime or launch failure";
    default: return "unknown status";
    }
}

int deltanet_pick_cp_groups(int B, int H, int T, int dk, int dv, int chunk) {
    const int st = check_shape(dk, dv, chunk, DN_BF16);
    if (st != DN_OK && check_shape(dk, dv, chunk, DN_F32) != DN_OK) return st;
    if (B <= 0 || H <= 0 || T < 0) return DN_ERR_INVALID;
    int G, cpg;
    resolve_groups(0, B, H, T, dv, G, cpg, fwd_lead_shape(dk, dv));
    return G;
}

size_t deltanet_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int cp_groups) {
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0) return 0;
    if (check_shape(dk, dv, chunk, DN_BF16) != DN_OK && check_shape(dk, dv, chunk, DN_F32) != DN_OK)
        return 0;
    int G, cpg;
    resolve_groups(cp_groups, B, H, T, dv, G, cpg, fwd_lead_shape(dk, dv));
    return ws_bytes_for(B, H, dk, dv, G);
}

int deltanet_fwd(const void *q, const void *k, const void *v, const void *beta, const float *S0,
                 void *o, float *S_final, int B, int H, int T, int dk, int dv, int chunk, int dtype,
                 int cp_groups, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return fwd_dense(q, k, v, beta, nullptr, S0, o, S_final, B, H, T, 1, dk, dv, chunk, dtype, cp_groups, workspace,
                     workspace_bytes, stream, true);
}

int deltanet_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                        const float *S0, void *o, float *S_final, const int32_t *cu_seqlens,
                        const int32_t *seq_order, int N, int total_T, int H, int dk, int dv,
                        int chunk, int dtype, hipStream_t stream) {
    return fwd_varlen(q, k, v, beta, nullptr, S0, o, S_final, cu_seqlens, seq_order, N, total_T, H, dk, dv, chunk,
                      dtype, stream);
}

int deltanet_gated_fwd(const void *q, const void *k, const void *v, const void *beta, const float *g,
                       const float *S0, void *o, float *S_final, int B, int H, int T, int dk, int dv,
                       int chunk, int dtype, int cp_groups, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (T > 0 && !g) return DN_ERR_INVALID;
    return fwd_dense(q, k, v, beta, g, S0, o, S_final, B, H, T, 1, dk, dv, chunk, dtype, cp_groups, workspace,
                     workspace_bytes, stream, true);
}

int deltanet_gdp_fwd(const void *q, const void *k, const void *v, const void *beta, const float *g,
                     const float *S0, void *o, float *S_final, int B, int H, int T, int n_h, int dk,
                     int dv, int chunk, int dtype, int cp_groups, void *workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (n_h <= 0 || T < 0) return DN_ERR_INVALID;
    if ((int64_t)T * n_h > INT32_MAX / 2) return DN_ERR_UNSUPPORTED;
    if (T > 0 && !g) return DN_ERR_INVALID;
    return fwd_dense(q, k, v, beta, g, S0, o, S_final, B, H, T * n_h, n_h, dk, dv, chunk, dtype, cp_groups,
                     workspace, workspace_bytes, stream, true);
}

int deltanet_gated_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                              const float *g, const float *S0, void *o, float *S_final,
                              const int32_t *cu_seqlens, const int32_t *seq_order, int N, int total_T,
                              int H, int dk, int dv, int chunk, int dtype, hipStream_t stream) {
    if (total_T > 0 && !g) return DN_ERR_INVALID;
    return fwd_varlen(q, k, v, beta, g, S0, o, S_final, cu_seqlens, seq_order, N, total_T, H, dk, dv, chunk, dtype,
                      stream);
}

int deltanet_kda_fwd(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
                     void *o, float *S_final, int B, int H, int T, int dk, int dv, int chunk, int dtype, int cp_groups,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_shape(dk, dv, chunk, dtype);
    if (st != DN_OK) return st;
    if (dtype != DN_BF16) return DN_ERR_UNSUPPORTED;
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0) return DN_ERR_INVALID;
    if ((int64_t)B * H > (int64_t)1 << 24) return DN_ERR_UNSUPPORTED;
    if (T > 0) {
        if (!q || !k || !v || !beta || !g || !o) return DN_ERR_INVALID;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(g) || !aligned_to(beta, 2))
            return DN_ERR_INVALID;
    }
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return DN_ERR_INVALID;
    int G, cpg;
    resolve_groups(cp_groups, B, H, T, dv, G, cpg, fwd_lead_shape(dk, dv));
    const size_t need = ws_bytes_for(B, H, dk, dv, G);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return DN_ERR_WORKSPACE;
    if (T == 0) { // no tokens: the final state is the initial one
        if (!S_final) return DN_OK;
        const size_t n = (size_t)B * H * dv * dk;
        const hipError_t e = S0 ? hipMemcpyAsync(S_final, S0, n * sizeof(float), hipMemcpyDeviceToDevice, stream)
                                : dn::launch_fill(S_final, n, 0.f, stream);
        return e == hipSuccess ? DN_OK : DN_ERR_HIP;
    }
    dn::ChainArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gk = g;
    a.o = o;
    a.S0 = S0;
    a.S_final = S_final;
    a.B = B;
    a.H = H;
    a.T = T;
    a.nh = 1;
    hipError_t err;
    if (G <= 1) {
        a.kind = dn::kDense;
        a.n_units = B * H;
        a.n_tiles = dv / dn::kRows;
        err = dn::launch_kda(dk, dv, true, a, stream);
        return err == hipSuccess ? DN_OK : DN_ERR_HIP;
    }
    // Context parallelism, as for deltanet_fwd: (i) each group's transition
    // (P_g from the identity with no values, Q_g from a zero state), (ii) the
    // prefix composition of the group maps, (iii) every group from its start.
    float *ws = static_cast<float *>(workspace);
    const size_t per = (size_t)B * H * G;
    a.ws_P = ws;
    a.ws_Q = a.ws_P + per * dk * dk;
    a.ws_S = a.ws_Q + per * dv * dk;
    a.G = G;
    a.chunks_per_group = cpg;
    // At dk = dv = 128 with three or more groups, group 0 runs from S0 beside
    // the transitions of groups 1..G-2, as in the dense forward (one workgroup
    // per CU here: the transitions' 64-row tiles take two rounds of the CUs
    // and group 0's workgroups fit in the second), and the output phase
    // covers groups 1..G-1.
    const bool lead = fwd_lead_shape(dk, dv) && G >= 3;
    const int first = lead ? 1 : 0;
    dn::ChainArgs a0 = a;
    a0.kind = dn::kCpOutput;
    a0.cp_count = 1;
    a0.cp_lead = 1;
    a0.S_final = nullptr;
    a0.n_units = B * H;
    a0.n_tiles = dv / dn::kRows;
    a.kind = dn::kCpTransition;
    a.cp_first = first;
    a.n_units = B * H * (G - 1 - first);
    a.n_tiles = dv / dn::kRows + dk / dn::kRows;
    if (lead) {
        err = launch_beside(
            stream, true, [&](hipStream_t s) { return dn::launch_kda(dk, dv, true, a0, s); },
            [&](hipStream_t s) { return dn::launch_kda(dk, dv, false, a, s); });
    } else {
        err = dn::launch_kda(dk, dv, false, a, stream);
    }
    if (err != hipSuccess) return DN_ERR_HIP;
    err = dn::launch_compose(dk, dv, a, stream);
    if (err != hipSuccess) return DN_ERR_HIP;
    a.kind = dn::kCpOutput;
    a.n_units = B * H * (G - first);
    a.n_tiles = dv / dn::kRows;
    err = dn::launch_kda(dk, dv, true, a, stream);
    return err == hipSuccess ? DN_OK : DN_ERR_HIP;
}

int deltanet_kda_fwd_varlen(const void *q, const void *k, const void *v, const void *beta, const float *g,
                            const float *S0, void *o, float *S_final, const int32_t *cu_seqlens,
                            const int32_t *seq_order, int N, int total_T, int H, int dk, int dv, int chunk,
                            int dtype, hipStream_t stream) {
    int st = check_shape(dk, dv, chunk, dtype);
    if (st != DN_OK) return st;
    if (dtype != DN_BF16) return DN_ERR_UNSUPPORTED;
    if (N <= 0 || H <= 0 || total_T < 0 || !cu_seqlens) return DN_ERR_INVALID;
    if ((int64_t)N * H > (int64_t)1 << 24) return DN_ERR_UNSUPPORTED;
    if (total_T > 0) {
        if (!q || !k || !v || !beta || !g || !o) return DN_ERR_INVALID;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(g) || !aligned_to(beta, 2))
            return DN_ERR_INVALID;
    }
    if (!aligned_to(cu_seqlens, 4) || (seq_order && !aligned_to(seq_order, 4))) return DN_ERR_INVALID;
    if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return DN_ERR_INVALID;
    dn::ChainArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gk = g;
    a.o = o;
    a.S0 = S0;
    a.S_final = S_final;
    a.cu_seqlens = cu_seqlens;
    a.seq_order = seq_order;
    a.kind = dn::kVarlen;
    a.nh = 1;
    a.B = N;
    a.H = H;
    a.T = total_T;
    a.n_units = N * H;
    a.n_tiles = dv / dn::kRows;
    return dn::launch_kda(dk, dv, true, a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

size_t deltanet_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (B <= 0 || H <= 0 || T < 0 || check_shape(dk, dv, chunk, DN_BF16) != DN_OK) return 0;
    const size_t slots = (size_t)B * H * ((T + dn::kChunk - 1) / dn::kChunk);
    return bwd_slot_bytes(dk, dv, false) * slots;
}

size_t deltanet_bwd_cp_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int cp_groups) {
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0 || check_shape(dk, dv, chunk, DN_BF16) != DN_OK) return 0;
    int G, cpg;
    resolve_groups(cp_groups, B, H, T, dv, G, cpg);
    return deltanet_bwd_workspace_bytes(B, H, T, dk, dv, chunk) + ws_bytes_for(B, H, dk, dv, G);
}

size_t deltanet_gated_bwd_cp_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int cp_groups) {
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0 || check_shape(dk, dv, chunk, DN_BF16) != DN_OK) return 0;
    int G, cpg;
    resolve_groups(cp_groups, B, H, T, dv, G, cpg);
    return deltanet_gated_bwd_workspace_bytes(B, H, T, dk, dv, chunk) + ws_bytes_for(B, H, dk, dv, G);
}

size_t deltanet_bwd_varlen_workspace_bytes(int N, int total_T, int H, int dk, int dv, int chunk) {
    if (N <= 0 || H <= 0 || total_T < 0 || check_shape(dk, dv, chunk, DN_BF16) != DN_OK) return 0;
    return bwd_slot_bytes(dk, dv, false) * varlen_max_slots(N, total_T, H) + align16((size_t)(N + 1) * sizeof(int32_t));
}

size_t deltanet_gated_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (B <= 0 || H <= 0 || T < 0 || check_shape(dk, dv, chunk, DN_BF16) != DN_OK) return 0;
    const size_t slots = (size_t)B * H * ((T + dn::kChunk - 1) / dn::kChunk);
    return bwd_slot_bytes(dk, dv, true) * slots;
}

size_t deltanet_gated_bwd_varlen_workspace_bytes(int N, int total_T, int H, int dk, int dv, int chunk) {
    if (N <= 0 || H <= 0 || total_T < 0 || check_shape(dk, dv, chunk, DN_BF16) != DN_OK) return 0;
    return bwd_slot_bytes(dk, dv, true) * varlen_max_slots(N, total_T, H) + align16((size_t)(N + 1) * sizeof(int32_t));
}

int deltanet_bwd(const void *q, const void *k, const void *v, const void *beta, const float *S0, const void *dO,
                 const float *dS_final, void *dq, void *dk_, void *dv_, void *dbeta, float *dS0, int B, int H, int T,
                 int dk, int dv, int chunk, int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B <= 0 || H <= 0 || T < 0) return DN_ERR_INVALID;
    const size_t need = deltanet_bwd_workspace_bytes(B, H, T, dk, dv, chunk);
    return bwd_common(q, k, v, beta, nullptr, S0, dO, dS_final, dq, dk_, dv_, dbeta, nullptr, dS0, nullptr, nullptr, B,
                      H, T, 1, dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream);
}

int deltanet_bwd_cp(const void *q, const void *k, const void *v, const void *beta, const float *S0, const void *dO,
                    const float *dS_final, void *dq, void *dk_, void *dv_, void *dbeta, float *dS0, int B, int H, int T,
                    int dk, int dv, int chunk, int dtype, int cp_groups, void *workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0) return DN_ERR_INVALID;
    const size_t need = deltanet_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups);
    return bwd_common(q, k, v, beta, nullptr, S0, dO, dS_final, dq, dk_, dv_, dbeta, nullptr, dS0, nullptr, nullptr, B,
                      H, T, 1, dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream, cp_groups);
}

int deltanet_gated_bwd(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
                       const void *dO, const float *dS_final, void *dq, void *dk_, void *dv_, void *dbeta, float *dg,
                       float *dS0, int B, int H, int T, int dk, int dv, int chunk, int dtype, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    if (B <= 0 || H <= 0 || T < 0) return DN_ERR_INVALID;
    if (T > 0 && (!g || !dg)) return DN_ERR_INVALID;
    const size_t need = deltanet_gated_bwd_workspace_bytes(B, H, T, dk, dv, chunk);
    return bwd_common(q, k, v, beta, g, S0, dO, dS_final, dq, dk_, dv_, dbeta, dg, dS0, nullptr, nullptr, B, H, T, 1,
                      dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream);
}

int deltanet_gated_bwd_cp(const void *q, const void *k, const void *v, const void *beta, const float *g,
                          const float *S0, const void *dO, const float *dS_final, void *dq, void *dk_, void *dv_,
                          void *dbeta, float *dg, float *dS0, int B, int H, int T, int dk, int dv, int chunk, int dtype,
                          int cp_groups, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B <= 0 || H <= 0 || T < 0 || cp_groups < 0) return DN_ERR_INVALID;
    if (T > 0 && (!g || !dg)) return DN_ERR_INVALID;
    const size_t need = deltanet_gated_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups);
    return bwd_common(q, k, v, beta, g, S0, dO, dS_final, dq, dk_, dv_, dbeta, dg, dS0, nullptr, nullptr, B, H, T, 1,
                      dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream, cp_groups);
}

size_t deltanet_gdp_bwd_workspace_bytes(int B, int H, int T, int n_h, int dk, int dv, int chunk) {
    if (n_h <= 0 || T < 0 || (int64_t)T * n_h > INT32_MAX / 2) return 0;
    return deltanet_gated_bwd_workspace_bytes(B, H, T * n_h, dk, dv, chunk);
}

int deltanet_gdp_bwd(const void *q, const void *k, const void *v, const void *beta, const float *g, const float *S0,
                     const void *dO, const float *dS_final, void *dq, void *dk_, void *dv_, void *dbeta, float *dg,
                     float *dS0, int B, int H, int T, int n_h, int dk, int dv, int chunk, int dtype, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    if (B <= 0 || H <= 0 || T < 0 || n_h <= 0) return DN_ERR_INVALID;
    if ((int64_t)T * n_h > INT32_MAX / 2) return DN_ERR_UNSUPPORTED;
    if (T > 0 && (!g || !dg)) return DN_ERR_INVALID;
    const size_t need = deltanet_gdp_bwd_workspace_bytes(B, H, T, n_h, dk, dv, chunk);
    return bwd_common(q, k, v, beta, g, S0, dO, dS_final, dq, dk_, dv_, dbeta, dg, dS0, nullptr, nullptr, B, H, T * n_h,
                      n_h, dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream);
}

int deltanet_gated_bwd_varlen(const void *q, const void *k, const void *v, const void *beta, const float *g,
                              const float *S0, const void *dO, const float *dS_final, void *dq, void *dk_, void *dv_,
                              void *dbeta, float *dg, float *dS0, const int32_t *cu_seqlens, const int32_t *seq_order,
                              int N, int total_T, int H, int dk, int dv, int chunk, int dtype, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (N <= 0 || H <= 0 || total_T < 0 || !cu_seqlens) return DN_ERR_INVALID;
    if (total_T > 0 && (!g || !dg)) return DN_ERR_INVALID;
    if (!aligned_to(cu_seqlens, 4) || (seq_order && !aligned_to(seq_order, 4))) return DN_ERR_INVALID;
    const size_t need = deltanet_gated_bwd_varlen_workspace_bytes(N, total_T, H, dk, dv, chunk);
    return bwd_common(q, k, v, beta, g, S0, dO, dS_final, dq, dk_, dv_, dbeta, dg, dS0, cu_seqlens, seq_order, N, H,
                      total_T, 1, dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream);
}

int deltanet_bwd_varlen(const void *q, const void *k, const void *v, const void *beta, const float *S0,
                        const void *dO, const float *dS_final, void *dq, void *dk_, void *dv_, void *dbeta, float *dS0,
                        const int32_t *cu_seqlens, const int32_t *seq_order, int N, int total_T, int H, int dk,
                        int dv, int chunk, int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (N <= 0 || H <= 0 || total_T < 0 || !cu_seqlens) return DN_ERR_INVALID;
    if (!aligned_to(cu_seqlens, 4) || (seq_order && !aligned_to(seq_order, 4))) return DN_ERR_INVALID;
    const size_t need = deltanet_bwd_varlen_workspace_bytes(N, total_T, H, dk, dv, chunk);
    return bwd_common(q, k, v, beta, nullptr, S0, dO, dS_final, dq, dk_, dv_, dbeta, nullptr, dS0, cu_seqlens,
                      seq_order, N, H, total_T, 1, dk, dv, chunk, dtype, workspace, workspace_bytes, need, stream);
}

int deltanet_decode_step(const void *q, const void *k, const void *v, const void *beta, const float *g,
                         float *S, void *o, int B, int H, int dk, int dv, int dtype, hipStream_t stream) {
    return decode_common(q, k, v, beta, g, nullptr, S, o, B, H, dk, dv, dtype, stream);
}

int deltanet_kda_decode_step(const void *q, const void *k, const void *v, const void *beta, const float *g,
                             float *S, void *o, int B, int H, int dk, int dv, int dtype, hipStream_t stream) {
    if (!g || !aligned16(g)) return DN_ERR_INVALID;
    return decode_common(q, k, v, beta, nullptr, g, S, o, B, H, dk, dv, dtype, stream);
}

} // extern "C"
