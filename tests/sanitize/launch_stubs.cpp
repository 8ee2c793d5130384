// Host stand-ins for the kernel launches and the few HIP runtime calls of the
// C-ABI layer, for a CPU build of api.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer. Every buffer in that build is host memory, and
// each stand-in reads every byte a kernel of that launch reads and writes
// every byte it writes, with the extents derived from the launch arguments
// exactly as the kernels derive them. An extent that the C-ABI layer sized or
// carved wrongly (a workspace too small for its layout, a pointer offset past
// the end) then shows up as an out-of-bounds access.
#include "dn_internal.h"

#include <cstdio>
#include <cstring>

namespace {

volatile unsigned char sink;
int launches = 0;

void rd(const void *p, size_t bytes) {
    if (!p || !bytes) return;
    const unsigned char *c = static_cast<const unsigned char *>(p);
    unsigned char acc = 0;
    for (size_t i = 0; i < bytes; ++i) acc ^= c[i];
    sink = acc;
}

void wr(void *p, size_t bytes) {
    if (!p || !bytes) return;
    std::memset(p, 0x3c, bytes);
}

size_t esz_of(int dtype) { return dtype == 1 ? 2 : 4; }

// Chunk slots of a packed batch: chunk_base[N] chunks, times H heads.
size_t varlen_slots(const dn::ChainArgs &a) {
    return a.chunk_base ? (size_t)a.chunk_base[a.B] * a.H : 0;
}

void chain_common(int dtype, int dk, int dv, bool write_o, const dn::ChainArgs &a, bool kda) {
    ++launches;
    const size_t e = kda ? 2 : esz_of(dtype);
    const size_t units = (size_t)a.B * a.H;
    const size_t nh = a.nh > 0 ? a.nh : 1;
    size_t steps, real;
    if (a.kind == dn::kVarlen) {
        rd(a.cu_seqlens, (size_t)(a.B + 1) * 4);
        rd(a.seq_order, a.seq_order ? (size_t)a.B * 4 : 0);
        steps = real = (size_t)a.T;
    } else {
        steps = (size_t)a.B * a.T;
        real = steps / nh;
    }
    rd(a.q, real * a.H * dk * e);
    rd(a.k, steps * a.H * dk * e);
    rd(a.v, steps * a.H * dv * e);
    rd(a.beta, steps * a.H * e);
    rd(a.g, a.g ? real * a.H * 4 : 0);
    rd(a.gk, a.gk ? steps * a.H * dk * 4 : 0);
    if (a.kind == dn::kCpTransition) {
        const size_t per = units * a.G;
        wr(a.ws_P, per * dk * dk * 4);
        wr(a.ws_Q, per * dv * dk * 4);
        return;
    }
    if (a.kind == dn::kCpOutput) rd(a.ws_S, units * a.G * dv * dk * 4);
    if (a.kind == dn::kCpOutput && a.cp_lead) wr(a.ws_S, units * a.G * dv * dk * 4);
    rd(a.S0, a.S0 ? units * dv * dk * 4 : 0);
    if (write_o) wr(a.o, real * a.H * dv * e);
    wr(a.S_final, a.S_final ? units * dv * dk * 4 : 0);
    if (a.S_chunks16) {
        const size_t slots = a.kind == dn::kVarlen ? varlen_slots(a)
                                                   : units * (((size_t)a.T + dn::kChunk - 1) / dn::kChunk);
        wr(a.S_chunks16, slots * dv * dk * 2);
        wr(a.T_chunks, a.T_chunks ? slots * dn::kChunk * dn::kChunk * 2 : 0);
    }
}

// The inputs every backward launch reads: token tensors and, packed, the
// sequence offsets; returns the token steps and the real tokens.
void bwd_inputs(int dk, int dv, const dn::BwdArgs &b, size_t &steps, size_t &real) {
    const size_t nh = b.nh > 0 ? b.nh : 1;
    const bool varlen = b.cu_seqlens != nullptr;
    steps = varlen ? (size_t)b.T : (size_t)b.B * b.T;
    real = varlen ? steps : steps / nh;
    rd(b.q, real * b.H * dk * 2);
    rd(b.k, steps * b.H * dk * 2);
    rd(b.beta, steps * b.H * 2);
    rd(b.dO, real * b.H * dv * 2);
    if (varlen) {
        rd(b.cu_seqlens, (size_t)(b.B + 1) * 4);
        rd(b.chunk_base, (size_t)(b.B + 1) * 4);
    }
}

} // namespace

int stub_launch_count() { return launches; }
void stub_set_capturing(bool c);

namespace dn {

hipError_t launch_chain(int dtype, int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t) {
    chain_common(dtype, dk, dv, write_o, a, false);
    return hipSuccess;
}

hipError_t launch_kda(int dk, int dv, bool write_o, const ChainArgs &a, hipStream_t) {
    chain_common(1, dk, dv, write_o, a, true);
    return hipSuccess;
}

hipError_t launch_compose(int dk, int dv, const ChainArgs &a, hipStream_t) {
    ++launches;
    const size_t per = (size_t)a.B * a.H * a.G;
    rd(a.ws_P, per * dk * dk * 4);
    rd(a.ws_Q, per * dv * dk * 4);
    rd(a.S0, a.S0 ? (size_t)a.B * a.H * dv * dk * 4 : 0);
    wr(a.ws_S, per * dv * dk * 4);
    return hipSuccess;
}

hipError_t launch_chunk_base(const int32_t *cu_seqlens, int N, int32_t *cb, hipStream_t) {
    ++launches;
    cb[0] = 0;
    for (int n = 0; n < N; ++n) cb[n + 1] = cb[n] + (cu_seqlens[n + 1] - cu_seqlens[n] + kChunk - 1) / kChunk;
    return hipSuccess;
}


hipError_t launch_bwd_rev(int dk, int dv, const BwdArgs &b, hipStream_t) {
    ++launches;
    size_t steps, real;
    bwd_inputs(dk, dv, b, steps, real);
    const size_t units = (size_t)b.B * b.H, slots = (size_t)b.max_slots;
    rd(b.seq_order, b.cu_seqlens && b.seq_order ? (size_t)b.B * 4 : 0);
    rd(b.dS_final, b.dS_final ? units * dv * dk * 4 : 0);
    rd(b.T_chunks, slots * kChunk * kChunk * 2);
    if (b.rev_kind == kRevCpAffine) { // only the group-start gradients C_g of groups 1..G-1
        wr(b.ws_C + units * dv * dk, units * (b.G - 1) * dv * dk * 4);
        return hipSuccess;
    }
    if (b.rev_kind == kRevCpRun) rd(b.ws_E, units * (b.G - 1) * dv * dk * 4);
    wr(b.G_chunks, slots * dv * dk * 2);
    wr(b.dv, steps * b.H * dv * 2);
    wr(b.dS0, b.dS0 ? units * dv * dk * 4 : 0);
    return hipSuccess;
}

hipError_t launch_compose_bwd(int dk, int dv, const BwdArgs &b, hipStream_t) {
    ++launches;
    const size_t units = (size_t)b.B * b.H, per = units * b.G;
    rd(b.ws_P, per * dk * dk * 4);
    rd(b.ws_C, per * dv * dk * 4);
    rd(b.dS_final, b.dS_final ? units * dv * dk * 4 : 0);
    wr(b.ws_E, units * (b.G - 1) * dv * dk * 4);
    return hipSuccess;
}

hipError_t launch_bwd_grad(int dk, int dv, const BwdArgs &b, hipStream_t) {
    ++launches;
    size_t steps, real;
    bwd_inputs(dk, dv, b, steps, real);
    const size_t slots = (size_t)b.max_slots;
    rd(b.v, steps * b.H * dv * 2);
    rd(b.S_chunks16, slots * dv * dk * 2);
    rd(b.G_chunks, slots * dv * dk * 2);
    rd(b.T_chunks, slots * kChunk * kChunk * 2);
    wr(b.dq, real * b.H * dk * 2);
    wr(b.dk, steps * b.H * dk * 2);
    wr(b.dbeta, steps * b.H * 2);
    return hipSuccess;
}

hipError_t launch_bwd(int dk, int dv, const BwdArgs &b, hipStream_t) {
    ++launches;
    const size_t nh = b.nh > 0 ? b.nh : 1;
    const bool varlen = b.cu_seqlens != nullptr;
    const size_t steps = varlen ? (size_t)b.T : (size_t)b.B * b.T;
    const size_t real = varlen ? steps : steps / nh;
    const size_t units = (size_t)b.B * b.H;
    const size_t slots = (size_t)b.max_slots;
    rd(b.q, real * b.H * dk * 2);
    rd(b.k, steps * b.H * dk * 2);
    rd(b.v, steps * b.H * dv * 2);
    rd(b.beta, steps * b.H * 2);
    rd(b.dO, real * b.H * dv * 2);
    rd(b.g, b.g ? real * b.H * 4 : 0);
    rd(b.dS_final, b.dS_final ? units * dv * dk * 4 : 0);
    if (varlen) {
        rd(b.cu_seqlens, (size_t)(b.B + 1) * 4);
        rd(b.chunk_base, (size_t)(b.B + 1) * 4);
        rd(b.seq_order, b.seq_order ? (size_t)b.B * 4 : 0);
    }
    rd(b.S_chunks16, slots * dv * dk * 2);
    rd(b.T_chunks, slots * kChunk * kChunk * 2);
    if (b.rev_kind == kRevCpAffine) { // the group-start gradients C_g of groups 1..G-1 only
        wr(b.ws_C + units * dv * dk, units * (b.G - 1) * dv * dk * 4);
        return hipSuccess;
    }
    if (b.rev_kind == kRevCpRun) rd(b.ws_E, units * (b.G - 1) * dv * dk * 4);
    wr(b.part, (size_t)b.n_tiles * slots * bwd_part_bytes(dk));
    wr(b.dq, real * b.H * dk * 2);
    wr(b.dk, steps * b.H * dk * 2);
    wr(b.dv, steps * b.H * dv * 2);
    wr(b.dbeta, steps * b.H * 2);
    wr(b.dg, b.dg ? real * b.H * 4 : 0);
    wr(b.dS0, b.dS0 ? units * dv * dk * 4 : 0);
    return hipSuccess;
}

hipError_t launch_fill(float *p, size_t n, float value, hipStream_t) {
    ++launches;
    for (size_t i = 0; i < n; ++i) p[i] = value;
    return hipSuccess;
}

hipError_t launch_decode(int dtype, int dk, const DecodeArgs &a, hipStream_t) {
    ++launches;
    const size_t e = esz_of(dtype), n = (size_t)a.n_units;
    rd(a.q, n * dk * e);
    rd(a.k, n * dk * e);
    rd(a.v, n * a.dv * e);
    rd(a.beta, n * e);
    rd(a.g, a.g ? n * 4 : 0);
    rd(a.gk, a.gk ? n * dk * 4 : 0);
    rd(a.S, n * a.dv * dk * 4);
    wr(a.S, n * a.dv * dk * 4);
    wr(a.o, n * a.dv * e);
    return hipSuccess;
}

} // namespace dn

extern "C" {
hipError_t hipGetDevice(int *deviceId) {
    *deviceId = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *pi, hipDeviceAttribute_t, int) {
    *pi = 256;
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t sizeBytes, hipMemcpyKind, hipStream_t) {
    ++launches;
    std::memcpy(dst, src, sizeBytes);
    return hipSuccess;
}
// the second stream of the context-parallel forward: handles that are never
// dereferenced; the caller's stream reads as captured after
// stub_set_capturing(true), which sends the forward down its one-stream path
static int side_objects[3];
static bool stub_capturing = false;
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *s) {
    *s = stub_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned int) {
    *s = reinterpret_cast<hipStream_t>(&side_objects[0]);
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned int) {
    static int n = 1;
    *e = reinterpret_cast<hipEvent_t>(&side_objects[n]);
    n = n == 1 ? 2 : 1;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
}

void stub_set_capturing(bool c) { stub_capturing = c; }
