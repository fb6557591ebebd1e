/*
 * linattn.h — C ABI of the MI355X (gfx950) causal linear-attention library.
 *
 * The library computes linear attention with the feature map
 *   phi(x) = elu(x) + 1            ("Transformers are RNNs", Katharopoulos et
 *                                   al. 2020, translated page "線性變換器",
 *                                   §3.2.1 eq.(7); alpha = 1)
 * in four forms:
 *   - causal:      o_i = phi(q_i)^T S_i / phi(q_i)^T z_i,
 *                  S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j)
 *                  (same page, §3.3 eq.(9)-(12); the mask j <= i is inclusive);
 *   - non-causal:  the same with the sums over every j = 1..N (§3.2 eq.(5)-(6));
 *   - causal backward: dq, dk, dv of the causal form (§3.3.1);
 *   - decode step: one step of the RNN form, state updated first and then read
 *                  (§3.4 eq.(16)-(20), without f_l and the residual);
 *   - other feature maps: the causal and non-causal forms with DPFP-nu or the
 *                  degree-2 polynomial map in place of elu + 1 (§3.2.1);
 *   - delta rule:  the fast-weight memory W (M x D) of "Linear Transformers Are
 *                  Secretly Fast Weight Programmers" (Schlag et al. 2021; news
 *                  summary, paragraphs on the update rule and normalisation):
 *                  kh = phi(k)/sum(phi(k)), qh = phi(q)/sum(phi(q)),
 *                  vbar = W kh, W += beta (v - vbar) kh^T, o = W qh,
 *                  over a sequence or as a single decode step.
 * No 1/sqrt(D) scaling and no epsilon is applied (the pages apply none to these
 * forms; phi > 0 keeps every denominator positive).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are DEVICE pointers, contiguous and row-major, owned by the caller:
 *   q, k : [B, H, N, D]    v, o : [B, H, N, M]     (element type = dtype)
 *   S    : [B, H, D, M]    z    : [B, H, D]         (always float32)
 *   W    : [B, H, M, D]    beta : [B, H, N]         (W float32; beta = dtype)
 * dtype is LINATTN_F32 (float) or LINATTN_BF16 (bfloat16 bits, uint16).
 * bf16 inputs are read exactly; accumulation and state are float32; a bf16
 * output is rounded to nearest even once, from float32.
 * (D, M) must be one of {32, 64} x {32, 64}.  B, H, N may be 0 (nothing to
 * compute); negative sizes are rejected, and so are N (or Lmax) above 2^30 and
 * B*H above 2^30.
 * stream: a hipStream_t passed as void* (NULL = the default stream).  All work
 * is enqueued on it asynchronously; the library never synchronises, never
 * allocates device memory and keeps no pointer after returning.
 *
 * Error behaviour: every call validates its arguments before enqueuing
 * anything and returns a linattn_status_t:
 *   LINATTN_ERR_NULL        a required pointer is NULL, or a pair that must be
 *                           given together (S0/z0, S_out/z_out) is half given;
 *   LINATTN_ERR_SHAPE       a size is negative or an element count overflows;
 *   LINATTN_ERR_DTYPE       dtype is not LINATTN_F32 / LINATTN_BF16;
 *   LINATTN_ERR_UNSUPPORTED (D, M) is outside the built set;
 *   LINATTN_ERR_ALIGN       a pointer is not 16-byte aligned (beta: not
 *                           aligned to its element size);
 *   LINATTN_ERR_ALIAS       an output overlaps an input it must not overlap
 *                           (a state output identical to its input is allowed);
 *   LINATTN_ERR_WORKSPACE   the workspace is NULL or smaller than required;
 *   LINATTN_ERR_HIP         a kernel launch failed (hipGetLastError).
 * Values are not checked: NaN/Inf propagate, beta outside [0,1] follows the
 * formula.  Device faults surface at the caller's next synchronisation.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LINATTN_ABI_VERSION 4  /* 2: deltanet_fwd takes a workspace; 3: the feature-map and softmax decode entry points;
                                  4: linattn_noncausal_fwd_noalloc */

/* Size of the library-owned device scratch behind linattn_noncausal_fwd_noalloc
 * (one copy per GPU the library runs on, held until the process ends). */
#define LINATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum { LINATTN_F32 = 0, LINATTN_BF16 = 1 } linattn_dtype_t;

typedef enum {
  LINATTN_OK = 0,
  LINATTN_ERR_NULL = 1,
  LINATTN_ERR_SHAPE = 2,
  LINATTN_ERR_DTYPE = 3,
  LINATTN_ERR_UNSUPPORTED = 4,
  LINATTN_ERR_ALIGN = 5,
  LINATTN_ERR_ALIAS = 6,
  LINATTN_ERR_WORKSPACE = 7,
  LINATTN_ERR_HIP = 8
} linattn_status_t;

/* Bytes of device workspace linattn_causal_fwd needs for this problem (0 when
 * none is needed).  Returns 0 also for invalid arguments, which the forward
 * call then rejects. */
size_t linattn_causal_workspace_bytes(int B, int H, int N, int D, int M, int dtype);

/* Causal linear attention, eq.(9)-(12): for every (b, h) and i = 1..N,
 *   S_i = S0 + sum_{j<=i} phi(k_j) v_j^T,  z_i = z0 + sum_{j<=i} phi(k_j),
 *   o_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
 * o:            [B,H,N,M] output, or NULL to compute the final state only.
 * S0, z0:       initial state (both NULL means zero, as eq.(16)-(17)); read only.
 * S_out, z_out: final state S_N, z_N (both NULL: not written).  S_out may be
 *               the same pointer as S0 (and z_out as z0) for an in-place carry.
 * ws, ws_bytes: device workspace of at least linattn_causal_workspace_bytes();
 *               contents need no initialisation and are clobbered.
 * o must not overlap q, k, v, S0, z0, S_out, z_out or ws. */
int linattn_causal_fwd(const void* q, const void* k, const void* v, void* o,
                       int B, int H, int N, int D, int M, int dtype,
                       const float* S0, const float* z0, float* S_out, float* z_out,
                       void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace linattn_causal_bwd needs (0 when none). */
size_t linattn_causal_bwd_workspace_bytes(int B, int H, int N, int D, int M, int dtype);

/* Backward of the causal form for a sequence that starts from a zero state:
 * given dO = dL/do, the gradients dq, dk, dv of L through eq.(9)-(12) and phi
 * (§3.3.1 states that they are cumulative sums computable in linear time and
 * constant memory, without printing them).  With a_i = dO_i / den_i and
 * b_i = -(dO_i . o_i) / den_i:
 *   dphi(q_i) = S_i a_i + z_i b_i,
 *   dphi(k_j) = sum_{i>=j} phi(q_i) (a_i . v_j + b_i),
 *   dv_j      = sum_{i>=j} (phi(q_i) . phi(k_j)) a_i,
 *   dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k).
 * q, k, dq, dk: [B,H,N,D]; v, dO, dv: [B,H,N,M], all in dtype; arithmetic is
 * float32 for both dtypes.  The forward output is recomputed, not an input.
 * ws, ws_bytes: device workspace of at least linattn_causal_bwd_workspace_bytes().
 * dq, dk, dv must not overlap each other, the inputs or ws. */
int linattn_causal_bwd(const void* q, const void* k, const void* v, const void* dO,
                       void* dq, void* dk, void* dv, int B, int H, int N, int D, int M, int dtype,
                       void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace linattn_noncausal_fwd needs (0 when none). */
size_t linattn_noncausal_workspace_bytes(int B, int H, int N, int D, int M, int dtype);

/* Non-causal (encoder) linear attention, eq.(5)-(6): with
 *   S = sum_{j=1..N} phi(k_j) v_j^T and z = sum_{j=1..N} phi(k_j),
 *   o_i = phi(q_i)^T S / phi(q_i)^T z for every i.
 * Self-attention only: queries and keys share the length N.
 * o must not overlap q, k, v or ws. */
int linattn_noncausal_fwd(const void* q, const void* k, const void* v, void* o,
                          int B, int H, int N, int D, int M, int dtype,
                          void* ws, size_t ws_bytes, void* stream);

/* linattn_noncausal_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * static device array of LINATTN_NOALLOC_SCRATCH_BYTES owned by the library,
 * so the caller passes only inputs and outputs.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).
 * Limit: the problem must fit the scratch, i.e.
 *   linattn_noncausal_workspace_bytes(B, H, N, D, M, dtype) <= LINATTN_NOALLOC_SCRATCH_BYTES
 * (at D = M = 64 that holds for B*H up to about 1000 heads at any N);
 * a larger problem returns LINATTN_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (concurrent streams, or several host threads) race and must be
 * serialised by the caller.  The scratch keeps whatever the last call left;
 * this path writes every part of it before reading it.  The first call on a
 * device looks up that device's copy (hipGetSymbolAddress); a failure there
 * returns LINATTN_ERR_HIP.  Other errors as linattn_noncausal_fwd. */
int linattn_noncausal_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                  int B, int H, int N, int D, int M, int dtype, void* stream);

/* One autoregressive step of the RNN form, eq.(18)-(20), for B*H independent
 * states, in place:
 *   S <- S + phi(k) v^T,  z <- z + phi(k),  o = phi(q)^T S / phi(q)^T z
 * (the output reads the state that already holds this step's token).
 * q, k: [B,H,D]; v, o: [B,H,M] (dtype); S: [B,H,D,M], z: [B,H,D] float32,
 * read and written in place.  o must not overlap q, k, v, S or z. */
int linattn_decode_step(const void* q, const void* k, const void* v, void* o,
                        float* S, float* z, int B, int H, int D, int M, int dtype,
                        void* stream);

/* Softmax attention decode step over a key/value cache: the "stateful softmax"
 * baseline the recurrent form is compared with ("Transformers are RNNs",
 * translated page, Appendix C.1), with the attention of §3.1 eq.(2):
 *   Kc[L] <- k, Vc[L] <- v,  o = softmax(q Kc[0..L]^T / sqrt(D)) Vc[0..L],
 * for B*H independent heads.  Its cost grows with L, unlike the fixed-size
 * state of linattn_decode_step.
 * q, k: [B,H,D]; v, o: [B,H,M]; Kc: [B,H,Lmax,D]; Vc: [B,H,Lmax,M], all in
 * dtype, caller-owned; rows 0..L-1 of the caches hold the earlier tokens and
 * row L is written.  0 <= L < Lmax (else LINATTN_ERR_SHAPE).  Arithmetic is
 * float32; o is rounded to dtype.  o must not overlap q, k, v, Kc or Vc; the
 * caches must not overlap each other or q, k, v. */
int softmax_decode_step(const void* q, const void* k, const void* v, void* o,
                        void* Kc, void* Vc, int B, int H, int L, int Lmax,
                        int D, int M, int dtype, void* stream);

/* Feature maps other than elu + 1 for linattn_fmap_fwd. */
typedef enum { LINATTN_FMAP_DPFP = 1, LINATTN_FMAP_POLY2 = 2 } linattn_fmap_t;

/* Feature dimension C of a map: 2 nu D for LINATTN_FMAP_DPFP (nu = 1, 2 or 3),
 * D^2 for LINATTN_FMAP_POLY2 (nu = 0); 0 for an unsupported map, nu or D. */
int linattn_fmap_dim(int fmap, int nu, int D);

/* Bytes of device workspace linattn_fmap_fwd needs (0 when none, or for invalid
 * arguments, which the call then rejects). */
size_t linattn_fmap_workspace_bytes(int B, int H, int N, int D, int M, int dtype, int fmap, int nu);

/* Linear attention with another feature map phi: R^D -> R^C ("Transformers are
 * RNNs", translated page, §3.2.1: any map of dimension C gives O(N C M) work):
 *   LINATTN_FMAP_DPFP, order nu in {1, 2, 3} (DPFP-nu of "Linear Transformers
 *     Are Secretly Fast Weight Programmers", news summary, DPFP paragraph;
 *     the formula is not printed there, this is the reading built):
 *     r = (relu(x), relu(-x)) in R^{2D},
 *     phi(x)_{(n-1) 2D + i} = r_i r_{(i+n) mod 2D},  i < 2D,  n = 1..nu;
 *   LINATTN_FMAP_POLY2, nu = 0 (degree-2 polynomial kernel, §3.2.1):
 *     phi(x)_{a D + b} = x_a x_b, so phi(q).phi(k) = (q.k)^2.
 * causal != 0: eq.(9)-(12) with this phi (inclusive mask), from the initial
 *   state (S0, z0) ([B,H,C,M] and [B,H,C] float32; both NULL means zero).
 * causal == 0: eq.(5)-(6) over all N keys; S0 and z0 must be NULL
 *   (LINATTN_ERR_UNSUPPORTED otherwise).
 * o:            [B,H,N,M] output, or NULL to compute the final state only.
 * S_out, z_out: the final (causal) or total (non-causal) state, [B,H,C,M] and
 *               [B,H,C] float32, or both NULL.  S_out may equal S0 (and z_out z0).
 * ws, ws_bytes: device workspace of at least linattn_fmap_workspace_bytes();
 *               contents need no initialisation and are clobbered.
 * Products and sums are float32 for both dtypes.  No epsilon is added: a row
 * whose weights are all zero (possible with DPFP when no query-key pair shares
 * an active pair of components) gives 0/0 = NaN.
 * Errors as for linattn_causal_fwd; an unknown fmap or nu is
 * LINATTN_ERR_UNSUPPORTED.  o must not overlap q, k, v, S0, z0, S_out, z_out or
 * ws. */
int linattn_fmap_fwd(const void* q, const void* k, const void* v, void* o,
                     int B, int H, int N, int D, int M, int dtype, int fmap, int nu, int causal,
                     const float* S0, const float* z0, float* S_out, float* z_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Delta-rule fast-weight memory over a sequence, for every (b, h), i = 1..N:
 *   kh = phi(k_i)/sum_c phi(k_i)_c,  qh = phi(q_i)/sum_c phi(q_i)_c,
 *   vbar = W kh,  W <- W + beta_i (v_i - vbar) kh^T,  o_i = W qh
 * (retrieve the value bound to the key, then store the convex combination
 * beta_i v_i + (1 - beta_i) vbar in its place; the output reads the updated W).
 * beta: [B,H,N] in dtype, used as given (no squashing).
 * W0: [B,H,M,D] float32 initial memory, NULL means zero.
 * W_out: [B,H,M,D] float32 final memory, or NULL; may equal W0.
 * ws, ws_bytes: device workspace of at least deltanet_workspace_bytes();
 *               contents need no initialisation and are clobbered.
 * The sequence runs in chunks of 64 tokens: per chunk the same recurrence is
 * solved exactly as a unit lower-triangular system in the values written,
 * (I + diag(beta) L) U = diag(beta) (V - Kh W0^T), L the strictly lower part of
 * Kh Kh^T, so that only W0 -> W0 + U^T Kh is sequential.  The workspace holds,
 * for every chunk, the normalised keys Kh and T = (I + diag(beta) L)^{-1} diag(beta)
 * (lower triangle), each as a bf16 head and tail (28 KiB per chunk at D = 64,
 * 20 KiB at D = 32), formed for all chunks in parallel before the sequential pass.
 * o must not overlap q, k, v, beta, W0, W_out or ws. */
int deltanet_fwd(const void* q, const void* k, const void* v, const void* beta, void* o,
                 int B, int H, int N, int D, int M, int dtype,
                 const float* W0, float* W_out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace deltanet_fwd needs (0 when none). */
size_t deltanet_workspace_bytes(int B, int H, int N, int D, int M, int dtype);

/* One autoregressive step of the delta-rule memory (the RNN form of
 * deltanet_fwd, for one token) for B*H independent memories, in place:
 *   kh = phi(k)/sum_c phi(k)_c,  qh = phi(q)/sum_c phi(q)_c,
 *   vbar = W kh,  W <- W + beta (v - vbar) kh^T,  o = W qh
 * ("Linear Transformers Are Secretly Fast Weight Programmers", news summary,
 * paragraphs on the update rule and normalisation; the output reads the
 * updated memory).  N steps of this call equal deltanet_fwd over N tokens.
 * q, k: [B,H,D]; v, o: [B,H,M]; beta: [B,H] (dtype, used as given);
 * W: [B,H,M,D] float32, read and written in place.
 * o must not overlap q, k, v, beta or W; W must not overlap q, k, v or beta. */
int deltanet_decode_step(const void* q, const void* k, const void* v, const void* beta, void* o,
                         float* W, int B, int H, int D, int M, int dtype, void* stream);

/* Static, human-readable name of a status code ("LINATTN_OK", ...). */
const char* linattn_status_str(int status);

/* LINATTN_ABI_VERSION of the built library. */
int linattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
