/*
 * osdn.h - C ABI of the MI355X (gfx950) OSDN / Gated DeltaNet-2 forward library
 * (libosdn.so).
 *
 * Method sources, cited by page title and section:
 *  [OSDN-it] "Riepilogo Tecnico: OSDN: Miglioramento della Regola Delta con
 *            Precondizionamento Online Provabile nell'Attenzione Lineare"
 *            (gist.science/it/paper/2605.13473), sections 2.1-2.3.
 *  [GDN2-it] "Riepilogo Tecnico: Gated DeltaNet-2"
 *            (gist.science/it/paper/2605.22791), method parts 1-3.
 * (The status codes and conventions below apply to the gdn2_* entry points
 * too.)
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller, contiguous, row-major, in the layouts stated below. The library
 *    allocates nothing, and calls are reentrant and thread-safe. Its one piece
 *    of process-global mutable state is the optional per-kernel timing record
 *    of osdn_kernel_timing / osdn_kernel_times (off by default; guarded by a
 *    lock); no compute call depends on it.
 *  - Inputs are read-only. Outputs are fully overwritten. Pointers marked
 *    "required" may be NULL only when the tensor has no elements (B*H*T = 0).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued asynchronously; the call returns without synchronising, so a
 *    device-side fault surfaces at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    non-zero status means nothing was launched (except OSDN_ERR_HIP, returned
 *    when the HIP runtime rejects a launch).
 *  - Non-finite inputs are not checked; they propagate within their own
 *    (batch, head) stream only.
 *  - Supported sizes: Dk, Dv in {32, 64, 128}; chunk in {16, 32, 64};
 *    B, H, T >= 0 (any T: a last chunk shorter than `chunk` is handled;
 *    T = 0 returns the initial state; B*H = 0 enqueues nothing). The fp32 path
 *    additionally needs the chunk working set to fit in one compute unit's LDS
 *    (see osdn_forward_supported); otherwise OSDN_ERR_UNSUPPORTED.
 */
#ifndef OSDN_H_
#define OSDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of q, k, v (and b, w for GDN-2) and of the output o. */
enum { OSDN_F32 = 0, OSDN_BF16 = 1 };

/* Status codes. */
enum {
  OSDN_OK = 0,
  OSDN_ERR_NULL_ARG = 1,     /* a required pointer is NULL                */
  OSDN_ERR_BAD_DIMS = 2,     /* B, H or T negative                        */
  OSDN_ERR_UNSUPPORTED = 3,  /* Dk, Dv, chunk or dtype has no kernel      */
  OSDN_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required   */
  OSDN_ERR_ALIASING = 5,     /* partial overlap of an input and an output */
  OSDN_ERR_HIP = 6           /* the HIP runtime rejected a launch         */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* osdn_strerror(int status);

/* 1 if (Dk, Dv, chunk, dtype) has a kernel instance on this build, else 0. */
int osdn_forward_supported(int Dk, int Dv, int chunk, int dtype);

/*
 * Device workspace, in bytes, that osdn_forward needs for these sizes
 * (0 if the sizes are invalid or unsupported, or the call needs none); its
 * contents are only meaningful during one call. chunk = 64: the phase-1
 * scratch (osdn_precond_workspace_bytes) followed by the phase-2 scratch
 * (osdn_chunk_workspace_bytes), since phase 2 then forms the preconditioned
 * keys itself. Other chunks: the preconditioned keys ([B,H,T,Dk] in the
 * storage dtype, rounded up to 256 bytes) followed by scratch shared by the
 * two phases (the larger of the two). osdn_forward places its regions by the
 * same rule, so this many bytes always cover what it touches.
 */
size_t osdn_forward_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                    int chunk, int dtype);

/*
 * OSDN forward: phase 1 (preconditioner scan) then phase 2 (chunked WY delta
 * rule with K~ = d*k in the chunk Gram matrix and intra-chunk scores).
 *
 * Per (batch b, head h), tokens t = 1..T ([OSDN-it] 2.1-2.3):
 *   a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~_t = d_t*k_t
 *   S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k~_t^T
 *   o_t = scale * S_t q_t                        (after the token-t update)
 *   d_{t+1} = r_t d_t + eta beta_t (1 - beta_t c)/n * a   (0 step if n = 0)
 * i.e. online gradient descent on h_t(d) = ((1 - beta<d,k^2>)^2 - 1)/(2||k||^2)
 * with the forgetting gate r (r = 1 when r is NULL).
 *
 *   q, k     [B,H,T,Dk]  dtype            (required)
 *   v        [B,H,T,Dv]  dtype            (required)
 *   beta     [B,H,T]     fp32             (required)
 *   r        [B,H,T]     fp32             (NULL: no forgetting gate)
 *   eta      scalar step size of the preconditioner learner
 *   d0       [B,H,Dk]    fp32             (NULL: all ones)
 *   S0       [B,H,Dv,Dk] fp32             (NULL: zeros)
 *   scale    readout scale (1.0 is the plain reading)
 *   o        [B,H,T,Dv]  dtype            (required)
 *   S_T      [B,H,Dv,Dk] fp32 final state (NULL: not written)
 *   d_T      [B,H,Dk]    fp32 preconditioner after the last token (NULL: not
 *                        written)
 *   rho      [B,H,T]     fp32 residual contraction ratio per token (NULL: not
 *                        computed): rho_t = f_t(S_t) / f_t(S_{t-1}) =
 *                        (1 - beta_t <d_t, k_t*k_t>)^2, f_t(S) = ||S k_t - v_t||^2/2
 *                        ([OSDN-it] section 3, Theorem 5.2)
 *   q_geo    [B,H]       fp32 geometric mean of rho over the T tokens of each
 *                        stream, exp(mean log rho) (1 when T = 0; NULL: not
 *                        computed) ([OSDN-it] section 4.2)
 *            rho and q_geo depend on the phase-1 inputs only; asking for
 *            either adds one pass over the keys after phase 1.
 *   workspace / workspace_bytes: device scratch of at least
 *            osdn_forward_workspace_bytes(...) bytes, 256-byte aligned.
 * S_T may be exactly S0 and d_T exactly d0 (in-place state update); any other
 * overlap between an output and an input returns OSDN_ERR_ALIASING.
 */
int osdn_forward(int B, int H, int T, int Dk, int Dv, int chunk, int dtype,
                 const void* q, const void* k, const void* v,
                 const float* beta, const float* r, float eta,
                 const float* d0, const float* S0, float scale,
                 void* o, float* S_T, float* d_T, float* rho, float* q_geo,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (work captured into HIP
 * graphs, tight serving loops, harnesses that forbid hipMalloc):
 * osdn_forward with the library's own static device scratch in place of a
 * caller workspace. Arguments, layouts, results and status codes as in
 * osdn_forward, without workspace / workspace_bytes. The scratch holds
 * OSDN_NOALLOC_SCRATCH_BYTES bytes per device (held from library load until
 * the process ends); sizes whose osdn_forward_workspace_bytes exceeds it
 * return OSDN_ERR_WORKSPACE before anything is launched. Nothing is
 * allocated: the first call on a device looks up that device's scratch
 * address once. Every call on one device shares that device's scratch and
 * leaves its contents behind (no call needs it cleared): calls that overlap
 * in time on one device (other streams, other threads) race on it and must
 * be ordered by the caller.
 */
#define OSDN_NOALLOC_SCRATCH_BYTES (128u << 20)
int osdn_forward_noalloc(int B, int H, int T, int Dk, int Dv, int chunk,
                         int dtype, const void* q, const void* k, const void* v,
                         const float* beta, const float* r, float eta,
                         const float* d0, const float* S0, float scale,
                         void* o, float* S_T, float* d_T, float* rho,
                         float* q_geo, void* stream);

/*
 * Device scratch, in bytes, that osdn_precond_scan needs (0 if the sizes are
 * invalid or T = 0): per chunk of 64 tokens and (batch, head), a fp32 record
 * of the gate prefix, the step sizes, the 64 x 64 matrix that maps the
 * chunk's entry preconditioner to its step sizes and the gate ratios that
 * carry each step to the chunk's end, plus that entry value.
 */
size_t osdn_precond_workspace_bytes(int B, int H, int T, int Dk, int dtype);

/*
 * Phase 1 alone ([OSDN-it] 2.2, first phase of the two-phase implementation):
 * writes the preconditioned keys k~_t = d_t*k_t ([B,H,T,Dk], dtype; NULL: not
 * written), d_T ([B,H,Dk] fp32; NULL: not written) and the residual ratios
 * rho and q_geo (as in osdn_forward; NULL: not computed). Reads only k, beta,
 * r, eta and d0, with the same meaning and layout as in osdn_forward.
 * workspace / workspace_bytes: device scratch of at least
 * osdn_precond_workspace_bytes(...) bytes, 256-byte aligned, not overlapping
 * any argument.
 */
int osdn_precond_scan(int B, int H, int T, int Dk, int dtype, const void* k,
                      const float* beta, const float* r, float eta,
                      const float* d0, void* ktilde, float* d_T, float* rho,
                      float* q_geo, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Phase 2 alone ([OSDN-it] 2.1-2.2, second phase): the chunkwise WY delta rule
 * with caller-supplied write keys, S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t)
 * ktilde_t^T, o_t = scale * S_t q_t. ktilde is [B,H,T,Dk] in the storage dtype
 * (for OSDN, the output of osdn_precond_scan; ktilde == k gives plain
 * DeltaNet). Other arguments as in osdn_forward; ktilde is an input and must
 * not overlap any output.
 * workspace / workspace_bytes: device scratch of at least
 * osdn_chunk_workspace_bytes(...) bytes, 256-byte aligned, not overlapping
 * any argument.
 */
int osdn_chunk_forward(int B, int H, int T, int Dk, int Dv, int chunk,
                       int dtype, const void* q, const void* k,
                       const void* ktilde, const void* v, const float* beta,
                       const float* S0, float scale, void* o, float* S_T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device scratch, in bytes, that osdn_chunk_forward needs (0 if the sizes
 * are invalid or T = 0): per chunk and (batch, head), the chunk's operands
 * that do not depend on the entry state ((2 Dk + Dv + chunk) x chunk
 * elements of the storage dtype).
 */
size_t osdn_chunk_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                  int chunk, int dtype);

/* 1 if (Dk, Dv, chunk, dtype) has a GDN-2 kernel instance, else 0. */
int gdn2_forward_supported(int Dk, int Dv, int chunk, int dtype);

/*
 * Gated DeltaNet-2 forward ([GDN2-it] method part 1, chunked as in part 3).
 * Per (batch b, head h), tokens t = 1..T, with state S of shape Dk x Dv:
 *   S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T
 *   o_t = scale * S_t^T q_t                       (after the token-t update)
 * alpha_t = exp(log_alpha_t) is a per-key-channel decay, b_t the erase gate
 * (per key channel), w_t the write gate (per value channel).
 *
 *   q, k       [B,H,T,Dk] dtype     (required)
 *   v          [B,H,T,Dv] dtype     (required)
 *   log_alpha  [B,H,T,Dk] fp32      (required; <= 0 for a decay)
 *   b          [B,H,T,Dk] dtype     (required)
 *   w          [B,H,T,Dv] dtype     (required)
 *   S0         [B,H,Dk,Dv] fp32     (NULL: zeros)
 *   o          [B,H,T,Dv] dtype     (required)
 *   S_T        [B,H,Dk,Dv] fp32     (NULL: not written)
 * Any log_alpha <= 0 is accepted ([GDN2-it] method part 3: the decay is
 * absorbed into the erase and write factors): inside a chunk each factor
 * gamma_t / gamma_i is split at 16-token block boundaries so that every
 * stored factor is at most 1, and a block whose own decay exceeds e^-60 in
 * some channel has its diagonal entries summed exactly, element by element.
 * S_T may be exactly S0; no other overlap is allowed.
 * workspace / workspace_bytes: device scratch of at least
 * gdn2_forward_workspace_bytes(...) bytes, 256-byte aligned, not overlapping
 * any argument.
 */
int gdn2_forward(int B, int H, int T, int Dk, int Dv, int chunk, int dtype,
                 const void* q, const void* k, const void* v,
                 const float* log_alpha, const void* b, const void* w,
                 const float* S0, float scale, void* o, float* S_T,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Device scratch, in bytes, that gdn2_forward needs (0 if the sizes are
 * invalid or T = 0): as for osdn_chunk_workspace_bytes plus, per chunk, the
 * decayed queries (Dk x chunk elements of the storage dtype) and the exit
 * decays (Dk fp32 values). */
size_t gdn2_forward_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                    int chunk, int dtype);

/* 1 if (Dk, Dv, chunk, dtype) has a gated-OSDN kernel instance, else 0 (the
 * sizes of gdn2_forward_supported). */
int osdn_gated_forward_supported(int Dk, int Dv, int chunk, int dtype);

/* Device workspace, in bytes, that osdn_gated_forward needs (0 if the sizes
 * are invalid or unsupported, or the call needs none). chunk = 64, where the
 * engine's layout with the preconditioned keys formed inside it fits (bf16 at
 * every supported Dk, Dv; fp32 at Dk = 32, and at Dk = 64 with Dv <= 64):
 * osdn_precond_workspace_bytes followed by gdn2_forward_workspace_bytes.
 * Otherwise the preconditioned keys ([B,H,T,Dk] in the storage dtype, rounded
 * up to 256 bytes), then scratch shared by the two phases (the larger of the
 * two). The call places its regions by the same rule. */
size_t osdn_gated_forward_workspace_bytes(int B, int H, int T, int Dk, int Dv,
                                          int chunk, int dtype);

/*
 * OSDN on a backbone with per-key-channel decay ([OSDN-it] section 4 runs
 * OSDN on Gated DeltaNet and Kimi Delta Attention backbones; the pages do not
 * print the combined rule). Reading taken: the decay acts on the memory
 * before the token's OSDN step, and the preconditioner learner is unchanged:
 *   S_t = S_{t-1} Diag(alpha_t) + beta_t (v_t - S_{t-1} Diag(alpha_t) k_t) k~_t^T
 *   o_t = scale * S_t q_t,  k~_t = d_t*k_t,  d as in osdn_forward,
 * alpha_t = exp(log_alpha_t) per key channel (a per-head scalar decay is the
 * case of equal channels). Arguments as in osdn_forward, plus
 *   log_alpha [B,H,T,Dk] fp32 (required; <= 0 for a decay, of any
 *             strength, as for gdn2_forward).
 * State [B,H,Dv,Dk] as in osdn_forward; S_T may be exactly S0 and d_T exactly
 * d0. Runs phase 1, then the chunked engine with the decay absorbed into the
 * keys (at chunk 64 the engine forms the preconditioned keys itself from the
 * phase-1 records; otherwise phase 1 writes them into the workspace).
 */
int osdn_gated_forward(int B, int H, int T, int Dk, int Dv, int chunk,
                       int dtype, const void* q, const void* k, const void* v,
                       const float* beta, const float* r, float eta,
                       const float* log_alpha, const float* d0,
                       const float* S0, float scale, void* o, float* S_T,
                       float* d_T, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Recurrent decode ([OSDN-it] section 1: constant-memory recurrent inference;
 * same token rule as osdn_forward): advances T tokens (typically 1) through
 * the token recurrence itself, reading the state once and updating it in
 * place. No workspace; B*H workgroups, each holding one (batch, head) state
 * in registers.
 *
 *   q, k     [B,H,T,Dk]  dtype            (required)
 *   v        [B,H,T,Dv]  dtype            (required)
 *   beta     [B,H,T]     fp32             (required)
 *   r        [B,H,T]     fp32             (NULL: no forgetting gate)
 *   eta      step size of the preconditioner learner
 *   log_alpha [B,H,T,Dk] fp32 per-key-channel decay of a gated backbone,
 *            applied to the state before each token's step as in
 *            osdn_gated_forward (NULL: no decay, plain OSDN)
 *   S        [B,H,Dv,Dk] fp32 IN/OUT: the state before the tokens on entry,
 *                        after them on return (required)
 *   d        [B,H,Dk]    fp32 IN/OUT: the preconditioner, likewise (required)
 *   scale    readout scale
 *   o        [B,H,T,Dv]  dtype            (required)
 * Output o_t and the final S, d equal osdn_forward(..., d0 = d, S0 = S) (or
 * osdn_gated_forward with log_alpha) up to rounding. T = 0 leaves S and d untouched. S, d and o must not overlap each
 * other or any input (OSDN_ERR_ALIASING). Dk, Dv in {32, 64, 128}.
 */
int osdn_decode(int B, int H, int T, int Dk, int Dv, int dtype,
                const void* q, const void* k, const void* v,
                const float* beta, const float* r, float eta,
                const float* log_alpha, float* S, float* d, float scale,
                void* o, void* stream);

/*
 * Gated DeltaNet-2 recurrent decode ([GDN2-it] method part 1, token form):
 * T tokens of the gdn2_forward rule with the state S ([B,H,Dk,Dv] fp32,
 * required) updated in place; q, k, v, log_alpha, b, w and o as in
 * gdn2_forward. T = 0 leaves S untouched. S and o must not overlap each other
 * or any input. Dk, Dv in {32, 64, 128}; no workspace.
 */
int gdn2_decode(int B, int H, int T, int Dk, int Dv, int dtype,
                const void* q, const void* k, const void* v,
                const float* log_alpha, const void* b, const void* w,
                float* S, float scale, void* o, void* stream);

/*
 * Backward of the OSDN forward: the reverse-mode adjoint of the token
 * recurrence of [OSDN-it] sections 2.1-2.3 (the memory update with the
 * preconditioned key k~ = d * k, and the online learner of d with its
 * forgetting gate), the same rule osdn_forward and osdn_decode compute.
 * Given the adjoints of the outputs it returns the gradient of
 *   L = sum <do, o> + <dS_T, S_T> + <dd_T, d_T>
 * with respect to every input, the phase-1 preconditioner scan included.
 *
 *   q, k, v, beta, r, eta, d0, S0, scale   as in osdn_forward (r NULL: ones;
 *            d0 NULL: ones; S0 NULL: zeros)
 *   dout     [B,H,T,Dv]  dtype of q       adjoint of o (required)
 *   dS_T     [B,H,Dv,Dk] fp32             adjoint of S_T (NULL: zero)
 *   dd_T     [B,H,Dk]    fp32             adjoint of d_T (NULL: zero)
 *   dq, dk   [B,H,T,Dk]  fp32 OUT         (required)
 *   dv       [B,H,T,Dv]  fp32 OUT         (required)
 *   dbeta    [B,H,T]     fp32 OUT         (required)
 *   dr       [B,H,T]     fp32 OUT         (required; the gradient at r = 1
 *                                          when r is NULL)
 *   deta     [B,H]       fp32 OUT         eta's gradient per (batch, head);
 *                                          a caller sums it (required)
 *   dd0      [B,H,Dk]    fp32 OUT         (required)
 *   dS0      [B,H,Dv,Dk] fp32 OUT         (required)
 *   workspace  device scratch of osdn_backward_workspace_bytes() bytes,
 *            256-byte aligned; caller-owned, contents on entry ignored:
 *            per token the residual v - S k and the preconditioner, the
 *            state every 64 tokens and after the last, and per token and
 *            32-row slice of the value channels that slice's sums over its
 *            rows (3 Dk + 4 floats)
 * Where a key is all zero the learner takes no step (as in the forward) and
 * no gradient flows through its step size. Gradients are fp32 whatever the
 * input dtype (bf16 inputs are widened; the recurrence runs in fp32). No
 * output may overlap another output, an input or the workspace
 * (OSDN_ERR_ALIASING). Dk, Dv in {32, 64, 128}. Three kernels: the forward
 * storing what the reverse needs and the reverse walk, each over B*H*Dv/32
 * workgroups (a 32-row slice of one (batch, head) state and its adjoint in
 * registers), then one wave per (batch, head) adding the slices' sums and
 * carrying the adjoint of the preconditioner.
 */
size_t osdn_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv);
int osdn_backward(int B, int H, int T, int Dk, int Dv, int dtype,
                  const void* q, const void* k, const void* v,
                  const float* beta, const float* r, float eta,
                  const float* d0, const float* S0, float scale,
                  const void* dout, const float* dS_T, const float* dd_T,
                  float* dq, float* dk, float* dv, float* dbeta, float* dr,
                  float* deta, float* dd0, float* dS0, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Gate-aware backward of osdn_gated_forward: the adjoint of OSDN on a
 * per-key-channel-decay backbone (the decay applied to the state before the
 * token's step, as in osdn_gated_forward; [OSDN-it] section 4 with the
 * preconditioner learner of sections 2.1-2.3). Arguments as in
 * osdn_backward, plus
 *   log_alpha  [B,H,T,Dk] fp32           the decay (required)
 *   dlog_alpha [B,H,T,Dk] fp32 OUT       its gradient (required)
 * workspace: osdn_gated_backward_workspace_bytes() bytes, 256-byte aligned,
 * caller-owned: per token the preconditioner, the state every 64 tokens and
 * after the last, one interval of min(T, 64) states per (batch, head) (the
 * reverse pass recomputes each interval from its stored state rather than
 * undo the decay), and per token and 32-row slice of the value channels
 * that slice's sums over its rows (4 Dk + 4 floats). Other rules as in
 * osdn_backward.
 */
size_t osdn_gated_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv);
int osdn_gated_backward(int B, int H, int T, int Dk, int Dv, int dtype,
                        const void* q, const void* k, const void* v,
                        const float* beta, const float* r, float eta,
                        const float* log_alpha, const float* d0,
                        const float* S0, float scale, const void* dout,
                        const float* dS_T, const float* dd_T, float* dq,
                        float* dk, float* dv, float* dbeta, float* dr,
                        float* deta, float* dlog_alpha, float* dd0,
                        float* dS0, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Gate-aware backward of gdn2_forward ([GDN2-it] method, part 1, and the
 * gate-aware backward of its method part 3, here in token form): the
 * gradient of L = sum <dout, o> + <dS_T, S_T> with respect to q, k, v, the
 * decay log_alpha, the erase gate b, the write gate w and S0.
 *
 *   q, k, v, log_alpha, b, w, S0, scale   as in gdn2_forward (S0 NULL: zeros)
 *   dout     [B,H,T,Dv]  dtype of q       (required)
 *   dS_T     [B,H,Dk,Dv] fp32             (NULL: zero)
 *   dq, dk, dlog_alpha, db  [B,H,T,Dk] fp32 OUT   (required)
 *   dv, dw   [B,H,T,Dv]  fp32 OUT         (required)
 *   dS0      [B,H,Dk,Dv] fp32 OUT         (required)
 *   workspace  gdn2_backward_workspace_bytes() bytes, 256-byte aligned,
 *            caller-owned: the state every 64 tokens and after the last, one
 *            interval of min(T, 64) states per (batch, head), and per token
 *            and 32-row value slice that slice's row sums (4 Dk + 4 floats)
 * No output may overlap another output, an input or the workspace. Dk, Dv in
 * {32, 64, 128}; gradients fp32 whatever the input dtype.
 */
size_t gdn2_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv);
int gdn2_backward(int B, int H, int T, int Dk, int Dv, int dtype,
                  const void* q, const void* k, const void* v,
                  const float* log_alpha, const void* b, const void* w,
                  const float* S0, float scale, const void* dout,
                  const float* dS_T, float* dq, float* dk, float* dv,
                  float* dlog_alpha, float* db, float* dw, float* dS0,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing for measurement harnesses. While enabled, every entry
 * point records a HIP event on its stream before and after each kernel it
 * launches (two event records per kernel; events are created on first use
 * and kept). osdn_kernel_timing(1) enables and clears the record,
 * osdn_kernel_timing(0) disables. The record is process-global (shared by
 * every thread and stream) and guarded by a lock; a harness that times one
 * stream should not run other calls meanwhile.
 */
void osdn_kernel_timing(int enable);

/*
 * Waits for the recorded events and reports, for each distinct kernel name
 * in first-launch order (at most `max`), its name (static storage), launch
 * count and mean duration in milliseconds; any output pointer may be NULL.
 * Returns the number of distinct kernels recorded, or -1 if the HIP runtime
 * fails. Kernel names: precond_prep, precond_chain, precond_ktilde,
 * precond_rho (phase 1), wy_prep, wy_prep_fused (phase 2 forming the
 * preconditioned keys itself), wy_scan (phase 2), gdn2_prep, gdn2_scan
 * (GDN-2), gated_prep, gated_prep_fused, gated_scan (OSDN on a decaying
 * backbone), osdn_decode, gdn2_decode (recurrent decode), osdn_bwd_record,
 * osdn_bwd, osdn_bwd_learner (backward), gated_bwd_record, gated_bwd,
 * gated_bwd_learner, gdn2_bwd_record, gdn2_bwd, gdn2_bwd_out (gate-aware
 * backward).
 */
int osdn_kernel_times(int max, const char** names, int* counts, float* mean_ms);

#ifdef __cplusplus
}
#endif

#endif /* OSDN_H_ */
