/*
 * flashbob.h - C ABI of the MI355X (gfx950) exact backward-over-backward (BoB)
 * of softmax attention.
 *
 * Method: "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax
 * Attention" (arXiv 2609.24089), Abstract. BoB is the exact derivative of the
 * attention first backward; two row-wise scalars fix every output through
 * affine maps, so the work runs as two tiled passes that never hold an N x N
 * tensor in device memory.
 *
 * Per head (b, h), with s = scale, P = softmax_rows(s Q K^T), O = P V and the
 * textbook first backward
 *     dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D),
 *     dQ = s dS K,  dK = s dS^T Q,  dV = P^T dO,
 * the library returns the gradients of the scalar
 *     L = <gQ, dQ> + <gK, dK> + <gV, dV>
 * with respect to Q, K, V and dO. LSE and D are differentiated through (they
 * are functions of the inputs). No dropout, no bias, no gradient for `scale`.
 * Attention is non-causal unless FLASHBOB_CAUSAL is passed to the *_ex entry
 * points (then query i attends to keys j <= i; the masked scores are -inf
 * constants, a reading beyond the abstract, which does not treat masks).
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous [B, H, N, d] arrays, d fastest, in device memory
 *     owned by the caller; the library allocates and frees nothing.
 *   - Inputs are read only. Outputs are fully overwritten. No output may
 *     overlap an input, the workspace or another output.
 *   - Every device pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; no host synchronisation happens inside the call and the
 *     library keeps no state between calls, so calls on different streams
 *     with disjoint buffers may run concurrently.
 *   - Supported: d in {32, 64, 96, 128}, and d = 256 with FLASHBOB_BF16 inputs;
 *     N >= 1 (any length, ragged tails masked);
 *     B, H >= 0 (B*H*N == 0 is a no-op returning FLASHBOB_OK);
 *     B*H*N*d < 2^62; dtype FLASHBOB_F32 or FLASHBOB_BF16.
 *   - Errors are negative return codes. Every argument check runs before any
 *     HIP call, so a rejected call touches no device state. A failed kernel
 *     launch returns FLASHBOB_ERR_HIP; flashbob_strerror then gives the HIP
 *     error text of the last failure on the calling thread.
 */
#ifndef FLASHBOB_H
#define FLASHBOB_H

#include <stddef.h>

/* Exported entry points (the library is built with hidden default
 * visibility, so only these are visible to a loader). */
#if defined(__GNUC__) || defined(__clang__)
#define FLASHBOB_API __attribute__((visibility("default")))
#else
#define FLASHBOB_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLASHBOB_F32 = 0,  /* inputs float32; all arithmetic float32 */
  FLASHBOB_BF16 = 1  /* inputs bfloat16; MFMA operands bf16, accumulation and row scalars float32 */
} flashbob_dtype;

enum {
  FLASHBOB_OK = 0,
  FLASHBOB_ERR_NULL = -1,           /* a required pointer is NULL */
  FLASHBOB_ERR_SHAPE = -2,          /* negative size, or B*H*N*d too large */
  FLASHBOB_ERR_UNSUPPORTED_D = -3,  /* d not in {32, 64, 96, 128} (or 256 with bf16 inputs) */
  FLASHBOB_ERR_UNSUPPORTED_N = -4,  /* reserved (no N is rejected today besides N < 0) */
  FLASHBOB_ERR_DTYPE = -5,          /* unknown dtype */
  FLASHBOB_ERR_ALIGN = -6,          /* a pointer is not 16-byte aligned */
  FLASHBOB_ERR_WORKSPACE = -7,      /* workspace smaller than flashbob_workspace_bytes */
  FLASHBOB_ERR_ALIAS = -8,          /* an output overlaps an input, the workspace or another output */
  FLASHBOB_ERR_SCALE = -9,          /* scale is not finite */
  FLASHBOB_ERR_FLAGS = -10,         /* unknown flag bits, or an empty or unknown stage set */
  FLASHBOB_ERR_SCRATCH = -11,       /* flashbob_bob_noalloc: B*H*N exceeds its static buffer */
  FLASHBOB_ERR_HIP = -100           /* a HIP call failed; see flashbob_strerror */
};

/* Flags of the *_ex entry points. */
enum {
  FLASHBOB_CAUSAL = 1,          /* query i attends to keys j <= i */
  FLASHBOB_FIRST_BACKWARD = 2,  /* flashbob_bob_ex only: also write the first backward dQ, dK, dV */
  FLASHBOB_SAVED_LSE = 4,       /* flashbob_bob_ex only: pass 1 starts from a saved log-sum-exp */
  FLASHBOB_BF16_OUTPUTS = 8     /* flashbob_bob_ex only: outputs are stored as bf16 */
};

/* Stage sets of flashbob_bob_ex (the three kernels of the schedule). */
enum {
  FLASHBOB_STAGE_PASS1 = 1,        /* row scalars into the workspace */
  FLASHBOB_STAGE_PASS2_QUERY = 2,  /* gradQ, graddO from the workspace's row scalars */
  FLASHBOB_STAGE_PASS2_KEY = 4,    /* gradK, gradV from the workspace's row scalars */
  FLASHBOB_STAGES_ALL = 7
};

/* Bytes of device workspace flashbob_bob needs: four float32 row-scalar
 * vectors [B, H, N] (LSE, D, c, r), rounded up to 256 bytes. Returns 0 for
 * B*H*N == 0 or for invalid (negative) sizes.
 * Source: FlashBoB (arXiv 2609.24089), Abstract: the first pass hands the
 * second one row statistics only, O(N) per head, never an N x N tensor. */
FLASHBOB_API size_t flashbob_workspace_bytes(int B, int H, int N, int d);

/* Exact BoB (the method's two-pass schedule: row scalars, then outputs).
 * Source: FlashBoB (arXiv 2609.24089), Abstract: exact differentiation
 * through the attention backward, organised as two passes over on-chip
 * tiles with no N x N intermediate in device memory.
 *   Q, K, V, dO      [B, H, N, d] inputs of the attention first backward
 *   gQ, gK, gV       [B, H, N, d] cotangents on its outputs dQ, dK, dV
 *                    (all seven in `dtype`)
 *   gradQ, gradK,
 *   gradV, graddO    [B, H, N, d] float32 outputs: dL/dQ, dL/dK, dL/dV, dL/ddO
 *   scale            softmax scale s (finite; commonly 1/sqrt(d))
 *   workspace        device buffer of at least flashbob_workspace_bytes(B,H,N,d)
 *                    bytes; its contents on entry do not matter and on return
 *                    hold the row scalars in the form pass 2 consumes,
 *                    (LSE * log2(e), -D, -c/s, -r) as [4][B][H][N] float32
 *                    (flashbob_rowstats returns them plainly).
 * Pass 1 (one kernel) computes the row scalars of every query. Pass 2
 * recomputes the score tiles and contracts them into the outputs in two
 * kernels: a query-major sweep producing gradQ and graddO and a key-major
 * sweep producing gradK and gradV, each accumulating in registers (no
 * atomics, so results are bitwise reproducible run to run). */
FLASHBOB_API int flashbob_bob(const void* Q, const void* K, const void* V, const void* dO,
                 const void* gQ, const void* gK, const void* gV,
                 float* gradQ, float* gradK, float* gradV, float* graddO,
                 int B, int H, int N, int d, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* The three kernels of flashbob_bob as separate calls, for callers that time
 * or schedule them individually. Source: FlashBoB (arXiv 2609.24089),
 * Abstract: the two passes of the schedule (the second split here into a
 * query-side and a key-side sweep). Same arguments and checks as flashbob_bob;
 * calling pass1, pass2_query and pass2_key in this order on one stream with
 * the same buffers is exactly flashbob_bob (the two pass-2 calls are
 * independent of each other).
 *   pass1:       writes the row scalars (pass-2 form, see above) into `workspace`;
 *                touches no output.
 *   pass2_query: reads the row scalars from `workspace`, writes gradQ and
 *                graddO (query-major sweep over the keys).
 *   pass2_key:   reads the row scalars from `workspace`, writes gradK and
 *                gradV (key-major sweep over the queries). */
FLASHBOB_API int flashbob_bob_pass1(const void* Q, const void* K, const void* V, const void* dO,
                       const void* gQ, const void* gK, const void* gV,
                       float* gradQ, float* gradK, float* gradV, float* graddO,
                       int B, int H, int N, int d, float scale, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
FLASHBOB_API int flashbob_bob_pass2_query(const void* Q, const void* K, const void* V, const void* dO,
                             const void* gQ, const void* gK, const void* gV,
                             float* gradQ, float* gradK, float* gradV, float* graddO,
                             int B, int H, int N, int d, float scale, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream);
FLASHBOB_API int flashbob_bob_pass2_key(const void* Q, const void* K, const void* V, const void* dO,
                           const void* gQ, const void* gK, const void* gV,
                           float* gradQ, float* gradK, float* gradV, float* graddO,
                           int B, int H, int N, int d, float scale, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* General form of flashbob_bob and of the three stage calls above.
 * Source: FlashBoB (arXiv 2609.24089), Abstract (the BoB itself); masks,
 * grouped heads, the first-backward outputs, a saved log-sum-exp and bf16
 * outputs are extensions beyond it:
 *   H_kv    key/value heads (grouped-query attention; H_kv = H is plain
 *           multi-head, H_kv = 1 multi-query). 1 <= H_kv <= H, H a multiple
 *           of H_kv. Q, dO, gQ, gradQ, graddO are [B, H, N, d]; K, V, gK, gV,
 *           gradK, gradV are [B, H_kv, N, d]; query head h uses key/value head
 *           h / (H / H_kv), and gradK, gradV sum over each group's query heads
 *           (the gradients of the shared heads). Otherwise FLASHBOB_ERR_SHAPE.
 *   flags   any of FLASHBOB_CAUSAL, FLASHBOB_FIRST_BACKWARD. Causal: per head,
 *           each query row i uses keys 0..i only; key blocks wholly above the
 *           diagonal are skipped, so the work is about half. First backward:
 *           dQ (float32, like gradQ) and dK, dV (float32, like gradK) also
 *           receive the first backward of the same attention (dQ = s dS K,
 *           dK = s dS^T Q, dV = P^T dO, summed over groups like gradK); dQ is
 *           written by the pass-2 query stage, dK and dV by the key stage. The
 *           extra products run in one-wave-per-SIMD variants of the pass-2
 *           kernels. Without the flag dQ, dK, dV are ignored (may be NULL).
 *           Saved LSE: lse_in ([B, H, N] float32, 4-byte aligned, an input
 *           that must not overlap any output) holds each query row's
 *           natural-log log-sum-exp of s Q K^T (masked like the call), as a
 *           forward pass saves it. Pass 1 then uses it as the row maximum for
 *           the whole sweep instead of tracking a running one, and still
 *           normalises by the sum it accumulates, so the result does not
 *           depend on lse_in being exact: values within 20 of the true ones
 *           give the same outputs up to rounding (far enough below them the
 *           exponentials overflow, far enough above they underflow). Without
 *           the flag lse_in is ignored (may be NULL).
 *           bf16 outputs: gradQ, gradK, gradV, graddO (and dQ, dK, dV) hold
 *           bf16 values (2 bytes per element, same shapes and 16-byte
 *           alignment): the float32 results rounded to nearest even as they
 *           are stored. The arithmetic is unchanged; the workspace and
 *           lse_in stay float32. Without the flag the outputs are float32.
 *   stages  a non-empty subset of FLASHBOB_STAGES_ALL, run in the order
 *           pass 1, pass 2 query side, pass 2 key side. Pass 2 stages read the
 *           row scalars pass 1 left in `workspace` (computed with the same
 *           flags and inputs).
 * Other arguments, checks and return codes as flashbob_bob; unknown flag
 * bits or stage sets return FLASHBOB_ERR_FLAGS. */
FLASHBOB_API int flashbob_bob_ex(const void* Q, const void* K, const void* V, const void* dO,
                    const void* gQ, const void* gK, const void* gV,
                    void* gradQ, void* gradK, void* gradV, void* graddO,
                    void* dQ, void* dK, void* dV, const float* lse_in,
                    int B, int H, int H_kv, int N, int d, float scale, int dtype, int flags, int stages,
                    void* workspace, size_t workspace_bytes, void* stream);

/* flashbob_bob without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The row scalars go to a static buffer
 * of the library instead: FLASHBOB_NOALLOC_SCRATCH_BYTES of device memory
 * that each GPU the library runs on holds until the process ends, enough for
 * B*H*N <= FLASHBOB_NOALLOC_MAX_ROWS query rows (larger calls return
 * FLASHBOB_ERR_SCRATCH before any HIP call). Everything else (arguments,
 * checks, results, asynchrony) is as flashbob_bob; results are bitwise equal
 * to flashbob_bob's. The buffer belongs to the device current on the
 * calling thread (its address is looked up on the first call there, the
 * only HIP call besides the kernel launches) and is shared by every call on
 * that device: calls that overlap on one GPU (other streams or threads)
 * race on it, so such callers serialise them. Nothing in it needs clearing:
 * pass 1 overwrites every value pass 2 reads. */
#define FLASHBOB_NOALLOC_MAX_ROWS (1 << 20)
#define FLASHBOB_NOALLOC_SCRATCH_BYTES (16u << 20)
FLASHBOB_API int flashbob_bob_noalloc(const void* Q, const void* K, const void* V, const void* dO,
                                      const void* gQ, const void* gK, const void* gV,
                                      float* gradQ, float* gradK, float* gradV, float* graddO,
                                      int B, int H, int N, int d, float scale, int dtype, void* stream);

/* Pass 1 alone (row statistics), exported for testing the first pass.
 * Source: FlashBoB (arXiv 2609.24089), Abstract: the two row-wise scalars
 * that fix every BoB output through affine maps (read as c and r below,
 * next to the first backward's D and the log-sum-exp).
 * Writes, per query row, LSE (natural-log log-sum-exp of s Q K^T), the
 * first-backward scalar D = rowsum(dO o O) and the two BoB row scalars
 *     c = rowsum(P o G),   r = rowsum(dS o G) + rowsum(P o H),
 * where G = s (gQ K^T + Q gK^T) and H = dO gV^T; each output is [B, H, N]
 * float32. Inputs as for flashbob_bob. */
FLASHBOB_API int flashbob_rowstats(const void* Q, const void* K, const void* V, const void* dO,
                      const void* gQ, const void* gK, const void* gV,
                      float* lse, float* D, float* c, float* r,
                      int B, int H, int N, int d, float scale, int dtype,
                      void* stream);

/* flashbob_rowstats with key/value heads H_kv (as for flashbob_bob_ex) and
 * flags (0 or FLASHBOB_CAUSAL; with the mask, the row scalars are those of the
 * causal attention). */
FLASHBOB_API int flashbob_rowstats_ex(const void* Q, const void* K, const void* V, const void* dO,
                         const void* gQ, const void* gK, const void* gV,
                         float* lse, float* D, float* c, float* r,
                         int B, int H, int H_kv, int N, int d, float scale, int dtype, int flags,
                         void* stream);

/* Static description of an error code; for FLASHBOB_ERR_HIP, the HIP error
 * text of the calling thread's last failure. Never NULL. (Library plumbing;
 * the method's pages define no error model.) */
FLASHBOB_API const char* flashbob_strerror(int code);

/* ABI version (major * 100 + minor). (Library plumbing.) */
FLASHBOB_API int flashbob_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHBOB_H */
