/*
 * deltanet.h -- C-ABI of the MI355X (gfx950) DeltaNet chunkwise forward pass.
 *
 * What is computed. For every (sequence, head) unit the library runs the
 * DeltaNet delta-rule recurrence, with the state S (dv x dk) acting on column
 * vectors:
 *     S_t = S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 * ("Linear Attention, Visualized", Haoran Zhang: DeltaNet > "Recurrent form",
 * with the state transposed as in "Context Parallelism for DeltaNet",
 * yywangcs, section 2). It evaluates that recurrence with the chunkwise
 * algorithm of the first page (DeltaNet > "Chunkwise algorithm" > "Complete
 * per-chunk algorithm"), chunk C = 64: per chunk r
 *     L = (K K^T) masked strictly lower,  (I + diag(beta) L) T = diag(beta),
 *     W = T K,  U = T V,  Z = U - W S_r^T,
 *     O_r = Q S_r^T + ((Q K^T) masked lower-inclusive) Z,
 *     S_{r+1} = S_r + Z^T K.
 * The readout is after the write (inclusive causal mask); q is not scaled;
 * q and k are used exactly as given (no normalisation inside).
 *
 * Gated DeltaNet (deltanet_gated_fwd*): the same page, section "Gated
 * DeltaNet (GDN)", adds a per-token scalar decay a_t of the previous state:
 *     S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
 * evaluated with that section's "Complete per-chunk algorithm": with
 * lambda[i:j] the product of a over chunk positions i..j, the masks of L and
 * of Q K^T take the factor lambda[i+1:l] at (l, i), K enters W with rows
 * scaled by lambda[1:l], Q enters the Q S^T part of O scaled by lambda[1:l],
 * and S_{r+1} = lambda[1:C] S_r + Z^T (K with rows scaled by lambda[l+1:C]).
 * The decay is passed as g_t = ln a_t (float32, the layout of beta); a_t = 1
 * (g_t = 0) gives DeltaNet. The kernels form prefix sums of g within each
 * chunk and only ever exponentiate differences with the later token first,
 * so every factor lies in (0, 1] for g <= 0. g must be finite; g > 0 (growth)
 * is accepted but may overflow.
 *
 * Context parallelism (cp_groups > 1) splits each unit's chunk chain into
 * groups. Each group first computes its affine map S_end = S_start P_g + Q_g
 * (P_g the ordered product of (I - W^T K) over its chunks, Q_g its state from
 * a zero start), a short pass composes these maps to fix every group's start
 * state, and then all groups produce their outputs in parallel ("Context
 * Parallelism for DeltaNet", sections 1-3; the chunk as an affine recurrence
 * in "Linear Attention, Visualized", DeltaNet > "One chunk as an affine
 * recurrence"). The result equals the serial one up to rounding.
 *
 * Layouts (row-major, contiguous, element strides fixed by the shape):
 *   q, k : [B, T, H, dk]    v, o : [B, T, H, dv]    beta, g : [B, T, H]
 *   S0, S_final : [B, H, dv, dk] float32 (S[b,h] is the dv x dk state)
 *   varlen: q, k [T_total, H, dk], v, o [T_total, H, dv], beta, g [T_total, H],
 *           S0/S_final [N, H, dv, dk]; sequence n owns tokens
 *           [cu_seqlens[n], cu_seqlens[n+1]) and starts from S0[n] (or zero).
 * q, k, v, beta and o share the element type `dtype`; g, S0 and S_final
 * are always float32. All arithmetic accumulates in float32; with DN_BF16 the
 * matrix-core operands are bfloat16 (intermediates W, T, Z and the state are
 * rounded to bfloat16 where they enter a matrix product; the state itself is
 * kept in float32).
 *
 * Supported shapes: chunk == 64; dk, dv in {64, 128} for DN_BF16; dk == 64,
 * dv in {64, 128} for DN_F32. Any T >= 0 (a partial last chunk is masked).
 *
 * Ownership and threading. Every pointer is device memory owned by the
 * caller. The library allocates nothing, frees nothing and never
 * synchronises: work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and completes asynchronously. The library keeps no state
 * between calls except a per-device cache of the compute-unit count, and is
 * safe to call from several threads. o and S_final must not overlap any input.
 *
 * Errors. Arguments are checked before anything is enqueued; on a non-zero
 * return nothing was launched and no output was written. Launch failures
 * return DN_ERR_HIP. Faults during execution surface at the caller's next
 * synchronisation of `stream`. NaN/Inf inputs are not detected; they
 * propagate.
 */
#ifndef DELTANET_H
#define DELTANET_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, beta and o. */
typedef enum { DN_F32 = 0, DN_BF16 = 1 } dn_dtype_t;

/* Status codes. */
enum {
    DN_OK = 0,
    DN_ERR_INVALID = -1,     /* NULL/misaligned pointer, negative or zero size, bad enum */
    DN_ERR_UNSUPPORTED = -2, /* valid request the library does not implement (chunk, dk, dv) */
    DN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than deltanet_workspace_bytes */
    DN_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

/*
 * Forward pass over B sequences of T tokens each.
 *   q, k, v, beta : inputs (see layouts above); required, 16-byte aligned.
 *   S0            : initial states [B,H,dv,dk] fp32, or NULL for zero states.
 *   o             : output [B,T,H,dv], required (may be NULL only when T == 0).
 *   S_final       : final states [B,H,dv,dk] fp32, or NULL to skip writing them.
 *   chunk         : must be 64.
 *   dtype         : DN_F32 or DN_BF16.
 *   cp_groups     : 1 = one serial chunk chain per unit; G > 1 = context
 *                   parallelism with G groups (clamped to the chunk count);
 *                   0 = let the library choose from the shape and the device's
 *                   compute-unit count (deltanet_pick_cp_groups).
 *   workspace, workspace_bytes : device scratch for cp_groups != 1; must hold
 *                   deltanet_workspace_bytes(...) bytes (may be NULL/0 when the
 *                   resolved group count is 1). Contents are scratch; they need
 *                   no initialisation and are clobbered.
 *   stream        : HIP stream to enqueue on. With context parallelism at
 *                   dk = dv = 128 (three or more groups) part of the call runs
 *                   on a second stream the library keeps per device, forked
 *                   from and joined back into `stream` with events, so the
 *                   call is still ordered on `stream` alone; while `stream`
 *                   is being captured everything runs on `stream`.
 * Returns DN_OK or a negative status.
 */
int deltanet_fwd(const void *q, const void *k, const void *v, const void *beta,
                 const float *S0, void *o, float *S_final, int B, int H, int T,
                 int dk, int dv, int chunk, int dtype, int cp_groups,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward pass over N packed sequences of different lengths.
 *   cu_seqlens : device int32 [N+1], cu_seqlens[0] = 0, non-decreasing,
 *                cu_seqlens[N] = total_T. Not validated on the device: values
 *                that break these rules give undefined results.
 *   seq_order  : device int32 [N], a permutation of 0..N-1 giving the order in
 *                which sequences are scheduled (longest first balances the
 *                load), or NULL for 0..N-1. Results do not depend on it.
 *   S0, S_final: [N,H,dv,dk] fp32 or NULL.
 * Other arguments as in deltanet_fwd. No workspace is needed.
 */
int deltanet_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                        const float *S0, void *o, float *S_final,
                        const int32_t *cu_seqlens, const int32_t *seq_order, int N,
                        int total_T, int H, int dk, int dv, int chunk, int dtype,
                        hipStream_t stream);

/*
 * Gated DeltaNet forward pass over B sequences of T tokens each
 * ("Gated DeltaNet (GDN)" > "Complete per-chunk algorithm", see above).
 *   g : log decays ln a_t, float32 [B,T,H], 4-byte aligned; required when T > 0.
 * Every other argument, the workspace (same size as deltanet_fwd's for the
 * same shape and cp_groups) and the error behaviour are as in deltanet_fwd.
 * Context parallelism applies unchanged: a group's chunks still map its
 * start state affinely to its end state.
 */
int deltanet_gated_fwd(const void *q, const void *k, const void *v, const void *beta,
                       const float *g, const float *S0, void *o, float *S_final, int B, int H,
                       int T, int dk, int dv, int chunk, int dtype, int cp_groups,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gated Delta Product forward pass ("Linear Attention, Visualized", "Gated
 * Delta Product (GDP)"): each real token t carries n_h (key, value, beta)
 * substeps applied in order after one decay of the previous state,
 *     S_{t,0} = a_t S_{t-1},  S_{t,j} = S_{t,j-1}(I - b_{t,j} k_{t,j} k_{t,j}^T) + b_{t,j} v_{t,j} k_{t,j}^T,
 *     S_t = S_{t,n_h},  o_t = S_t q_t,
 * evaluated as Gated DeltaNet over the virtual sequence of T n_h steps of
 * that page's "GDP as GDN over a virtual sequence" (decay on the first
 * substep, query on the last). The kernels index real tokens directly; no
 * virtual copy of q, g or o is made.
 *   q    : [B, T, H, dk]          k : [B, T, n_h, H, dk]     v : [B, T, n_h, H, dv]
 *   beta : [B, T, n_h, H]         g : [B, T, H] float32 (required when T > 0)
 *   o    : [B, T, H, dv]          S0, S_final : [B, H, dv, dk] float32
 * k, v and beta in this layout are already in virtual order. n_h >= 1
 * (n_h = 1 is deltanet_gated_fwd). Workspace: deltanet_workspace_bytes with
 * T n_h in place of T. Other arguments and errors as in deltanet_gated_fwd.
 */
int deltanet_gdp_fwd(const void *q, const void *k, const void *v, const void *beta,
                     const float *g, const float *S0, void *o, float *S_final, int B, int H,
                     int T, int n_h, int dk, int dv, int chunk, int dtype, int cp_groups,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gated DeltaNet forward pass over N packed sequences.
 *   g : log decays, float32 [T_total, H]; required when total_T > 0.
 * Other arguments as in deltanet_fwd_varlen.
 */
int deltanet_gated_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                              const float *g, const float *S0, void *o, float *S_final,
                              const int32_t *cu_seqlens, const int32_t *seq_order, int N,
                              int total_T, int H, int dk, int dv, int chunk, int dtype,
                              hipStream_t stream);

/*
 * One decode step: one new token per (sequence, head) applied to a state held
 * in HBM, in place ("Linear Attention, Visualized": DeltaNet > "Recurrent
 * form", one step of the recurrence above; with g, one step of "Gated
 * DeltaNet (GDN)"). For each unit u = (b, h):
 *     S[u] <- a S[u] (I - beta k k^T) + beta v k^T,   o = S[u] q   (a = exp(g); 1 if g is NULL)
 *   q, k : [B, H, dk]   v, o : [B, H, dv]   beta : [B, H]   (element type dtype)
 *   g    : [B, H] float32 log decays, or NULL for DeltaNet
 *   S    : [B, H, dv, dk] float32, read and overwritten (e.g. the S_final of a
 *          forward pass, which continues exactly from there)
 * dk, dv in {64, 128} for both dtypes. Alignment: q and k to 4 elements, S to
 * 16 bytes, the others to their element size. o must not overlap S or the
 * inputs. Errors as in deltanet_fwd. No workspace.
 */
int deltanet_decode_step(const void *q, const void *k, const void *v, const void *beta,
                         const float *g, float *S, void *o, int B, int H, int dk, int dv,
                         int dtype, hipStream_t stream);

/*
 * Kimi Delta Attention forward ("Linear Attention, Visualized", "Kimi Delta
 * Attention (KDA)"), DN_BF16 only: the previous state decays per key
 * channel, then the delta correction applies:
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
 * with a_t = exp(g_t) elementwise (state transposed as above).
 *   g : [B, T, H, dk] float32 log decays, 16-byte aligned, required when T > 0.
 * Evaluated with that section's complete per-chunk algorithm on sub-chunks of
 * 16 tokens (exact for any chunk size). Any decay a in (0, 1] per channel is
 * supported: where a channel decays by more than 2^96 within a sub-chunk, the
 * in-sub-chunk products take each pair's own decay factor instead of the
 * factored form (exact, slower; decays below fp32's range act as a reset).
 * Other arguments as in deltanet_fwd, including context
 * parallelism (cp_groups, with deltanet_workspace_bytes of workspace): each
 * group's transition is the same kernel run from the identity with no values,
 * which the per-channel decay leaves a linear map of the entering state.
 */
int deltanet_kda_fwd(const void *q, const void *k, const void *v, const void *beta,
                     const float *g, const float *S0, void *o, float *S_final, int B, int H,
                     int T, int dk, int dv, int chunk, int dtype, int cp_groups, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * deltanet_kda_fwd over a packed batch of N sequences (layouts as in
 * deltanet_fwd_varlen: tokens [total_T, H, *], g [total_T, H, dk] float32,
 * cu_seqlens [N + 1], optional seq_order, S0 / S_final [N, H, dv, dk]); the
 * state starts afresh at each sequence. DN_BF16 only.
 */
int deltanet_kda_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                            const float *g, const float *S0, void *o, float *S_final,
                            const int32_t *cu_seqlens, const int32_t *seq_order, int N,
                            int total_T, int H, int dk, int dv, int chunk, int dtype,
                            hipStream_t stream);

/*
 * One Kimi Delta Attention decode step (the recurrence above for a single
 * token), in place, for every unit u = (b, h):
 *     S[u] <- S[u] Diag(exp(g)) (I - beta k k^T) + beta v k^T,   o = S[u] q
 *   g : [B, H, dk] float32 per-channel log decays, 16-byte aligned (required)
 * Other arguments, dtypes, shapes and errors as in deltanet_decode_step; the
 * state continues exactly from deltanet_kda_fwd's S_final.
 */
int deltanet_kda_decode_step(const void *q, const void *k, const void *v, const void *beta,
                             const float *g, float *S, void *o, int B, int H, int dk, int dv,
                             int dtype, hipStream_t stream);

/*
 * Backward pass of deltanet_fwd (DN_BF16 only): gradients for upstream dO of
 * the output and dS_final of the final state. The pages give no backward
 * pass; this is the chain rule applied to the per-chunk algorithm above (see
 * the kernels' notes), exact up to rounding, with bf16 matrix-core operands
 * and fp32 accumulation.
 *   q, k, v, beta, S0 : the forward inputs (S0 NULL: zero)
 *   dO      : [B,T,H,dv] (dtype);  dS_final : [B,H,dv,dk] fp32 or NULL (zero)
 *   dq, dk, dv, dbeta : outputs, layouts of q, k, v, beta (dtype)
 *   dS0     : [B,H,dv,dk] fp32 output, or NULL to skip
 *   workspace : at least deltanet_bwd_workspace_bytes(...) bytes, 16-byte
 *             aligned: per chunk, the state entering it and the gradient of
 *             the state leaving it (bf16 each) and its T (as the forward pass
 *             forms it)
 * Three launches: the forward chain keeping the per-chunk states, the reverse
 * chain of the state gradient (dv, dS0), and a chunk-parallel pass for dq,
 * dk, dbeta. Errors as in deltanet_fwd (DN_ERR_UNSUPPORTED for DN_F32, and
 * for H > 65536).
 */
int deltanet_bwd(const void *q, const void *k, const void *v, const void *beta,
                 const float *S0, const void *dO, const float *dS_final, void *dq, void *dk,
                 void *dv, void *dbeta, float *dS0, int B, int H, int T, int dk_, int dv_,
                 int chunk, int dtype, void *workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Bytes of workspace deltanet_bwd needs (0 for invalid shapes). */
size_t deltanet_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * deltanet_bwd with the chunk chains split into cp_groups contiguous groups
 * of chunks per sequence (1: serial, as deltanet_bwd; 0: the library's choice,
 * deltanet_pick_cp_groups less the forward's extra group at dk = dv = 128),
 * for long sequences with few (sequence, head)
 * units. Over a group the reverse chain is affine in the gradient at the
 * group's end, dS_start = dS_end P_g^T + C_g, with P_g the group's forward
 * transition ("Context Parallelism for DeltaNet", section 2, the affine group
 * map, taken in reverse mode; the pages give no backward pass). The forward
 * states come from the context-parallel forward (transitions of every group,
 * their composition, every group from its start state); the reverse chain
 * then forms C_g of groups 1..G-1 from a zero end gradient, composes the end
 * gradients of all groups from dS_final, and runs every group from its own.
 * Results match deltanet_bwd up to rounding. Arguments as deltanet_bwd;
 * workspace: at least deltanet_bwd_cp_workspace_bytes(...) bytes, 16-byte
 * aligned (deltanet_bwd's, plus per (sequence, head, group) P_g^T, and two
 * dv x dk fp32 matrices). cp_groups < 0: DN_ERR_INVALID.
 */
int deltanet_bwd_cp(const void *q, const void *k, const void *v, const void *beta,
                    const float *S0, const void *dO, const float *dS_final, void *dq, void *dk,
                    void *dv, void *dbeta, float *dS0, int B, int H, int T, int dk_, int dv_,
                    int chunk, int dtype, int cp_groups, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of workspace deltanet_bwd_cp needs for cp_groups (0 for invalid shapes). */
size_t deltanet_bwd_cp_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int cp_groups);

/*
 * deltanet_bwd over a packed batch of N sequences (layouts as in
 * deltanet_fwd_varlen: tokens [total_T, H, *], cu_seqlens [N + 1] int32,
 * optional seq_order [N]; S0, dS_final, dS0 [N, H, dv, dk]); the state and
 * its gradient restart at each sequence. Workspace: at least
 * deltanet_bwd_varlen_workspace_bytes(...) bytes, 16-byte aligned, which
 * bounds the chunk count by total_T / 64 + N so the lengths need not be read
 * on the host. Errors as in deltanet_bwd.
 */
int deltanet_bwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                        const float *S0, const void *dO, const float *dS_final, void *dq,
                        void *dk, void *dv, void *dbeta, float *dS0, const int32_t *cu_seqlens,
                        const int32_t *seq_order, int N, int total_T, int H, int dk_,
                        int dv_, int chunk, int dtype, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Bytes of workspace deltanet_bwd_varlen needs (0 for invalid shapes). */
size_t deltanet_bwd_varlen_workspace_bytes(int N, int total_T, int H, int dk, int dv, int chunk);

/*
 * Backward pass of deltanet_gated_fwd (nh = 1, DN_BF16 only): the chain rule
 * on "Linear Attention, Visualized", "Gated DeltaNet (GDN)" > "Complete
 * per-chunk algorithm" (the pages give no backward pass), exact up to rounding.
 * Arguments as deltanet_bwd, plus
 *   g  : [B,T,H] fp32 log decays (the forward's), 4-byte aligned
 *   dg : [B,T,H] fp32 output, their gradient
 * Inside a chunk the decays enter through the row factors exp(gamma_t) and
 * exp(gamma_C - gamma_t) and the pairwise factors exp(gamma_t - gamma_s)
 * (gamma: in-chunk prefix sums of g), so g should be <= 0 (decay) as in the
 * forward; dg is the in-chunk suffix sum of the gradients of those prefix
 * sums. Workspace: at least deltanet_gated_bwd_workspace_bytes(...) bytes,
 * 16-byte aligned: per chunk, the state entering it (bf16), per 64 value rows
 * the chunk's sums over those rows (bf16, with fp32 per-token decay terms),
 * and its T. Errors as in deltanet_bwd; g or dg NULL with tokens present:
 * DN_ERR_INVALID.
 */
int deltanet_gated_bwd(const void *q, const void *k, const void *v, const void *beta,
                       const float *g, const float *S0, const void *dO, const float *dS_final,
                       void *dq, void *dk, void *dv, void *dbeta, float *dg, float *dS0, int B,
                       int H, int T, int dk_, int dv_, int chunk, int dtype, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_gated_bwd needs (0 for invalid shapes). */
size_t deltanet_gated_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * deltanet_gated_bwd with context parallelism, as deltanet_bwd_cp is to
 * deltanet_bwd: the decayed group map S -> S P_g + Q_g is still affine, so the
 * reverse chain over a group is affine in the gradient at its end with the
 * same P_g^T. Arguments as deltanet_gated_bwd plus cp_groups (1 serial, 0 the
 * library's choice); workspace: at least deltanet_gated_bwd_cp_workspace_bytes.
 */
int deltanet_gated_bwd_cp(const void *q, const void *k, const void *v, const void *beta,
                          const float *g, const float *S0, const void *dO, const float *dS_final,
                          void *dq, void *dk, void *dv, void *dbeta, float *dg, float *dS0, int B,
                          int H, int T, int dk_, int dv_, int chunk, int dtype, int cp_groups,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_gated_bwd_cp needs for cp_groups (0 for invalid shapes). */
size_t deltanet_gated_bwd_cp_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int cp_groups);

/*
 * deltanet_gated_bwd over a packed batch (layouts as in deltanet_bwd_varlen;
 * g, dg [total_T, H] fp32). Workspace: at least
 * deltanet_gated_bwd_varlen_workspace_bytes(...) bytes, 16-byte aligned.
 */
int deltanet_gated_bwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                              const float *g, const float *S0, const void *dO,
                              const float *dS_final, void *dq, void *dk, void *dv, void *dbeta,
                              float *dg, float *dS0, const int32_t *cu_seqlens,
                              const int32_t *seq_order, int N, int total_T, int H, int dk_,
                              int dv_, int chunk, int dtype, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_gated_bwd_varlen needs (0 for invalid shapes). */
size_t deltanet_gated_bwd_varlen_workspace_bytes(int N, int total_T, int H, int dk, int dv,
                                                 int chunk);

/*
 * Backward pass of deltanet_gdp_fwd (DN_BF16 only): "Linear Attention,
 * Visualized", "Gated Delta Product (GDP)" > "GDP as GDN over a virtual
 * sequence" makes GDP Gated DeltaNet over n_h substeps per token, so this is
 * the gated backward over that virtual sequence. Layouts as deltanet_gdp_fwd:
 *   q, dO : [B,T,H,dk] / [B,T,H,dv] (dtype), per real token (the query and the
 *           output sit on the last substep)
 *   k, v, beta : [B,T,n_h,H,*] per substep;  g : [B,T,H] fp32 (on the first substep)
 *   dq, dk, dv, dbeta, dg : outputs in the layouts of q, k, v, beta, g
 *   S0, dS_final, dS0 : as deltanet_gated_bwd
 * Workspace: at least deltanet_gdp_bwd_workspace_bytes(...) bytes, 16-byte
 * aligned (that of deltanet_gated_bwd at T n_h tokens). Errors as in
 * deltanet_gated_bwd; n_h <= 0: DN_ERR_INVALID; T n_h > 2^30: DN_ERR_UNSUPPORTED.
 */
int deltanet_gdp_bwd(const void *q, const void *k, const void *v, const void *beta,
                     const float *g, const float *S0, const void *dO, const float *dS_final,
                     void *dq, void *dk, void *dv, void *dbeta, float *dg, float *dS0, int B,
                     int H, int T, int n_h, int dk_, int dv_, int chunk, int dtype,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace deltanet_gdp_bwd needs (0 for invalid shapes). */
size_t deltanet_gdp_bwd_workspace_bytes(int B, int H, int T, int n_h, int dk, int dv, int chunk);

/*
 * deltanet_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation). The context-parallel workspace lives in a fixed
 * device array of the library, DN_NOALLOC_SCRATCH_BYTES (32 MiB) per device,
 * held from the first call on a device until the process ends; the call
 * itself allocates nothing. Semantics, layouts and errors as deltanet_fwd;
 * a shape and cp_groups whose deltanet_workspace_bytes exceeds
 * DN_NOALLOC_SCRATCH_BYTES returns DN_ERR_WORKSPACE before anything is
 * enqueued (cp_groups = 1 needs no workspace at any size). Every call on one
 * device shares that array: calls that overlap in time on one device (other
 * streams, other threads) race and must be serialised by the caller.
 */
#define DN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int deltanet_fwd_noalloc(const void *q, const void *k, const void *v, const void *beta,
                         const float *S0, void *o, float *S_final, int B, int H, int T,
                         int dk, int dv, int chunk, int dtype, int cp_groups, hipStream_t stream);

/*
 * Bytes of workspace deltanet_fwd (or deltanet_gated_fwd, deltanet_gdp_fwd,
 * deltanet_kda_fwd) needs for this
 * shape and cp_groups (0 means the library's choice on the current device).
 * Returns 0 when the resolved group count is 1, and also for invalid shapes.
 */
size_t deltanet_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                int cp_groups);

/*
 * Group count deltanet_fwd (and deltanet_gated_fwd, deltanet_gdp_fwd,
 * deltanet_kda_fwd) uses when called with cp_groups = 0, for the current HIP
 * device. Returns 1 (serial) when splitting does not pay, or a negative
 * status for invalid shapes. At dk = dv = 128 these forwards run group 0,
 * whose start state is S0, beside the transitions of the other groups (on a
 * second stream of the library, joined back into the caller's stream before
 * the call's later work; on the caller's stream itself while it is being
 * captured), so their choice there holds one group more than the choice of
 * the context-parallel backward passes with cp_groups = 0.
 */
int deltanet_pick_cp_groups(int B, int H, int T, int dk, int dv, int chunk);

/* Static, human-readable text for a status code. */
const char *deltanet_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DELTANET_H */
