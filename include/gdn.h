/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated-delta-rule forward library.
 *
 * The operation (per head, per sequence):
 *
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t,                 alpha_t = exp(g_t),
 *
 * the delta rule "change = rate x (target - prediction) x input" of HyMo's
 * "Model Architecture Walkthrough", section 5.2.2, with rate beta_t, target
 * v_t, input (write key) k_t and prediction alpha_t S_{t-1} k_t, after the
 * per-head scalar decay exp(g_t) of sections 5.2.1 and 5.3.1 of that page.
 * The read o_t uses the state after the step's write (section 5.2.1 reads
 * H_t); no 1/sqrt(dk) scale is applied.  The tensor layout follows the
 * pages' kernel interface: q, k are (B,T,H,dk), v and out are (B,T,H,dv),
 * g and beta are (B,T,H) ("Optimization Quartet", section 3.2 and the
 * wrapper of section 3.3), math in fp32, output in the caller's dtype.
 *
 * All pointers are DEVICE pointers on the current HIP device unless stated.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GDN_OK 0
#define GDN_ERR_INVALID_ARG (-1) /* null required pointer, bad size, bad dtype/chunk */
#define GDN_ERR_UNSUPPORTED (-2) /* valid request this build has no kernel for      */
#define GDN_ERR_LAUNCH (-3)      /* the HIP launch itself failed                      */
#define GDN_ERR_SCRATCH (-4)     /* too large for gdn_bwd_noalloc's fixed scratch      */

/* Storage dtype of q, k, v and out. */
#define GDN_F32 0
#define GDN_BF16 1

/* gdn_fwd flags. */
#define GDN_FLAG_NO_SEGMENTS 1 /* never cut a sequence into segments (see gdn_fwd) */

/*
 * gdn_fwd -- forward pass of the gated delta rule, chunkwise-parallel form.
 *
 * Dense mode (cu_seqlens == NULL): B sequences of T tokens each.
 *   q, k : (B, T, H, dk)   dtype         row-major, contiguous
 *   v    : (B, T, H, dv)   dtype
 *   g    : (B, T, H)       float32       natural-log decay, alpha = exp(g)
 *   beta : (B, T, H)       float32       write strength
 *   out  : (B, T, H, dv)   dtype         written; rounded to nearest even for bf16
 *
 * Packed mode (cu_seqlens != NULL): B sequences packed back to back,
 *   T = total tokens; q, k, v, g, beta, out drop the leading B dimension
 *   ((T, H, .) and (T, H)).  cu_seqlens is a DEVICE int32 array of B+1
 *   non-decreasing offsets with cu_seqlens[0] == 0 and cu_seqlens[B] == T;
 *   sequence n is tokens [cu_seqlens[n], cu_seqlens[n+1]).  Each sequence is
 *   an independent recurrence with its own initial and final state; chunks
 *   restart at each sequence start.  These device-side preconditions are not
 *   checked (checking would need a device read); violating them is undefined.
 *
 * State, both modes:
 *   h0   : (B, H, dk, dv)  float32, or NULL for a zero initial state.
 *   hT   : (B, H, dk, dv)  float32, written with the final state.
 *   hT[b,h,i,j] = S[j,i]: i runs over the key dimension, j over the value
 *   dimension (the pages' hidden state is (key dim) x (value dim)).
 *   hT may alias h0 exactly (in-place state update); out must not alias
 *   any input.  A sequence of length 0 gets hT = h0 (or zeros).
 *
 * Sizes: B >= 0, T >= 0, H >= 1, B*T < 2^31 tokens.  dk, dv in {32, 64, 128}.
 * dtype: GDN_F32 or GDN_BF16.
 * chunk: tokens per chunk; 0 selects 64 for GDN_BF16 and 16 for GDN_F32.
 *        GDN_BF16 accepts 32 and 64; GDN_F32 accepts 16 and 32 (64-token
 *        fp32 tiles exceed the 160 KB of LDS).  The result does not depend
 *        on the chunk length beyond floating-point rounding.
 * stream: a hipStream_t (NULL = the null stream).
 * flags: 0 or GDN_FLAG_NO_SEGMENTS; any other bit is GDN_ERR_INVALID_ARG.
 *
 * Pointers: q, k, v, g, beta and out are required when T > 0 and may be
 * NULL when T == 0 (no tokens); hT is required when B > 0.
 *
 * Behaviour: validates every host-side argument first; on any error returns
 * a negative status, launches nothing and leaves the outputs untouched.  On
 * success the work is queued on `stream` and the call returns GDN_OK
 * immediately; results are valid once the stream has been synchronised.
 * The caller owns all buffers; the library allocates no device memory,
 * keeps no pointer after returning and holds no global mutable state
 * (re-entrant, thread-safe).  Identical inputs give bitwise-identical
 * outputs on one device (no atomics, fixed reduction order).
 *
 * Segments.  Unless flags holds GDN_FLAG_NO_SEGMENTS, a long sequence may
 * run as several segments, one workgroup each: a segment starts from a
 * zero state at the latest chunk boundary behind it where the product of
 * the per-token transition norms exp(g) max(1, |1 - beta |k|^2|) is below
 * e^-40 (or at the sequence start, from h0), so it differs from the exact
 * sequential result by less than that factor of the state, beyond
 * rounding.  With GDN_BF16, dk = dv = 128 and 64-token chunks, a sequence
 * of n chunks is cut into ceil(n / 16) segments of equal length, but into
 * no more segments than the device has CUs per head (CUs / H, at least 1),
 * whatever the batch: a packed sequence's slice of out and hT then equals
 * the same sequence run alone (same H, h0 and flags, same device) bit for
 * bit.  Other GDN_BF16 shapes cut only dense batches with fewer chains x
 * 32-column tiles than the device has workgroup slots (the cut then depends
 * on the device), and never cut packed batches.  GDN_F32 never cuts.  hT == h0 turns cutting
 * off (a segment could read h0 after another wrote hT over it).  With
 * GDN_FLAG_NO_SEGMENTS every chain runs from its start, and a run split at
 * a chunk boundary (the second part taking the first part's hT as h0)
 * equals the whole run bit for bit.  Arithmetic: bf16 operands
 * with fp32 accumulation for GDN_BF16, fp32 throughout for GDN_F32; the
 * state is carried in fp32.  Non-finite inputs propagate.
 */
int gdn_fwd(const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* h0, const int32_t* cu_seqlens,
            void* out, float* hT, int B, int T, int H, int dk, int dv,
            void* stream, int dtype, int chunk, int flags);

/*
 * gdn_fwd_scan -- gdn_fwd with exact segment starts: the chunk-map scan.
 *
 * Over any run of chunks the rule is affine in the state: with M = S^T,
 * M_end = P M_start + Q, where P (dk x dk) depends on k, g and beta alone and
 * Q (dk x dv) is the end state reached from zero.  The chunkwise form of the
 * pages carries the state across chunks in series ("v1.0 Architecture &
 * Design Spec", section 2.3; "Optimization Quartet", section 3.2); composing
 * the chunks' maps lets a long sequence's segments run in parallel without
 * any dependence on decay.  A sequence of n > 16 chunks is cut as in gdn_fwd
 * (ceil(n / 16) segments of equal length, at most CUs / H of them) and run
 * in three launches on
 * `stream`:
 *   1. every segment but the last composes its map -- the recurrence over
 *      its chunks from the identity with v = 0 gives P, from zero with the
 *      real v gives Q (the first segment's Q starts from h0 and so is the
 *      second segment's entry state, and its P is not formed);
 *   2. a scan per chain gives the exact entry states, S_0 = h0,
 *      S_1 = Q_0, S_{s+1} = P_s S_s + Q_s (fp32, matrix cores);
 *   3. every segment runs the forward pass from S_s and stores its outputs;
 *      the last writes hT.
 * Unlike gdn_fwd's halo segments, the result does not depend on the decay
 * beyond rounding: a sequence with no decay at all is cut just the same.
 * It costs about three passes over each cut sequence instead of one, so
 * gdn_fwd is the faster choice when the decay makes halos short.
 *
 * Arguments, layouts, state semantics, error behaviour and determinism are
 * gdn_fwd's (flags are not taken), plus:
 *   workspace        DEVICE buffer of at least gdn_fwd_scan_workspace_size
 *                    bytes, 16-byte aligned, owned by the caller and used
 *                    only until the stream passes the call's last launch;
 *                    may be NULL when that size is 0.
 *   workspace_bytes  its size; too small (or a NULL / misaligned buffer
 *                    when one is needed) is GDN_ERR_INVALID_ARG.
 * After the call the workspace holds, for every segment slot sigma and head
 * h, three fp32 dk x dv row-major matrices at float offset
 * ((sigma * H + h) * 3 + m) * dk * dv: m = 0 the segment's P (m = 1 its Q,
 * m = 2 its entry state S), written only for segments of cut sequences
 * (P for segments 1 .. nseg-2, Q for 0 .. nseg-2, S for all).  Segment s of
 * dense sequence b is slot b * nseg + s; of packed sequence n, slot
 * floor(cu_seqlens[n] / 1024) + n + s (the workspace size counts the slots
 * without the CUs-per-head cap, so it does not depend on the device).
 * hT may alias h0: a cut sequence reads h0 only in the first two launches,
 * and an uncut one reads it in the same workgroup that later writes its hT.
 * A packed sequence's results equal the same sequence run alone bit for bit.
 * Shapes other than GDN_BF16 with dk = dv = 128 and 64-token chunks need no
 * workspace and run gdn_fwd with GDN_FLAG_NO_SEGMENTS (exact, uncut).
 */
long long gdn_fwd_scan_workspace_size(int B, int T, int H, int dk, int dv,
                                      int packed, int dtype, int chunk);
int gdn_fwd_scan(const void* q, const void* k, const void* v, const float* g,
                 const float* beta, const float* h0, const int32_t* cu_seqlens,
                 void* out, float* hT, int B, int T, int H, int dk, int dv,
                 void* stream, int dtype, int chunk, void* workspace,
                 long long workspace_bytes);

/*
 * gdn_fwd_recurrent -- the same operation in its token-by-token form, for
 * decoding and other short sequences: per token one rank-1 state update,
 *
 *   alpha = exp(g_t),  p = S_{t-1} k_t,
 *   S_t = alpha S_{t-1} + beta_t (v_t - alpha p) k_t^T,  o_t = S_t q_t,
 *
 * with the state kept on chip for the whole sequence ("Model Architecture
 * Walkthrough", sections 6.2-6.4, the read-after-write order of section
 * 5.2.1).  Arguments, layouts (dense and packed), state semantics, aliasing,
 * ownership, error behaviour and determinism are those of gdn_fwd; there is
 * no chunk argument.  Arithmetic is fp32 throughout (bf16 storage is widened
 * on load and the output rounded to nearest even), so for bf16 storage the
 * result differs from gdn_fwd's by the latter's bf16 operand rounding.  The
 * work per token is sequential, so gdn_fwd is the faster choice once a
 * sequence spans more than a few dozen tokens; this form's traffic is one
 * read of h0 and one write of hT per chain plus a single pass over the
 * tokens.
 */
int gdn_fwd_recurrent(const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* h0,
                      const int32_t* cu_seqlens, void* out, float* hT,
                      int B, int T, int H, int dk, int dv, void* stream,
                      int dtype);

/*
 * gdn_diag_fwd -- the diagonal-decay additive recurrence that HyMo writes
 * for its GDN layer, chunkwise form, with the block's epilogue fused:
 *
 *   H_t = exp(g_t A) (.) H_{t-1} + b_t (x) v_t,   A = -exp(A_log[h, :]),
 *   o_t = (c_t^T H_t + D_h v_t) * gate_t,
 *
 * per head, with the state H of shape (S, D): every key row s decays by its
 * own factor exp(g_t A_s), the write key b_t and value v_t add an outer
 * product (nothing is erased), and the read key c_t reads the state after
 * the write ("Model Architecture Walkthrough", section 5.2.1; the epilogue
 * of section 5.5 step 6 and section 5.6; the tensor layout of
 * "Optimization Quartet", section 3.2).
 *
 * Dense mode (cu_seqlens == NULL): B sequences of T tokens each.
 *   v    : (B, T, H, D)  dtype      values
 *   b, c : (B, T, H, S)  dtype      write and read keys
 *   g    : (B, T, H)     float32    per-head gate, g >= 0 (the pages' g is
 *                                   a sigmoid output); the chunkwise form
 *                                   relies on it (every decay factor <= 1)
 *   A_log: (H, S)        float32    A = -exp(A_log), one rate per key row
 *   Dskip: (H,)          float32    skip weight D_h, or NULL (no skip term)
 *   gate : (B, T, H)     float32    output gate, or NULL (no gate)
 *   out  : (B, T, H, D)  dtype      written (bf16: round to nearest even)
 * Packed mode (cu_seqlens != NULL): as for gdn_fwd -- the same tensors
 *   without the leading B, cu_seqlens a DEVICE int32 array of B+1 offsets
 *   (not checked on the device); each sequence is its own recurrence.
 * State: h0 (B, H, S, D) float32 or NULL (zero); hT (B, H, S, D) float32,
 *   hT[b,h,s,d] = H[s,d] after the sequence's last token; hT may alias h0
 *   exactly; a sequence of length 0 gets hT = h0 (or zeros).
 *
 * This form supports dtype GDN_BF16 with S = D = 32 (the pages' layer) and
 * chunk 0 or 64; other valid requests return GDN_ERR_UNSUPPORTED (the
 * token-by-token entry point below takes every size and both dtypes).
 * Sizes: B >= 0, T >= 0, H >= 1, (T + 64) * H * 64 < 2^31 bytes.
 * Pointers: v, b, c, g, A_log, out are required when T > 0; hT when B > 0.
 * Behaviour, ownership, stream semantics and determinism are those of
 * gdn_fwd.  Arithmetic: bf16 MFMA operands (keys scaled by their decays, the
 * state rounded to bf16 only as an operand) with fp32 accumulation; the
 * state is carried in fp32 and decays are formed in fp32.  The products of
 * per-token decays inside 16-token blocks use fp16 operands with fp32
 * accumulation, so |b| and |c| must stay below 65504 (the fp16 range);
 * a decay product below 2^-24 counts as zero there.
 */
int gdn_diag_fwd(const void* v, const void* b, const void* c, const float* g,
                 const float* A_log, const float* Dskip, const float* gate,
                 const float* h0, const int32_t* cu_seqlens, void* out, float* hT,
                 int B, int T, int H, int S, int D, void* stream, int dtype,
                 int chunk);

/*
 * gdn_diag_fwd_recurrent -- the same operation token by token, for decoding
 * and short sequences: per token alpha_s = exp(g_t A_s), H <- alpha (.) H +
 * b_t v_t^T, o_t = (c_t^T H + D_h v_t) * gate_t, with the state kept on chip
 * for the whole sequence (the loop the pages describe, "Model Architecture
 * Walkthrough", sections 5.5 step 5 and 6.2-6.4).  Arguments, layouts,
 * state semantics, aliasing and error behaviour are those of gdn_diag_fwd
 * without the chunk; any g is accepted.  S and D in {16, 32, 64, 128};
 * dtype GDN_F32 or GDN_BF16; arithmetic fp32 throughout (bf16 storage
 * widened on load, output rounded to nearest even).
 */
int gdn_diag_fwd_recurrent(const void* v, const void* b, const void* c,
                           const float* g, const float* A_log,
                           const float* Dskip, const float* gate,
                           const float* h0, const int32_t* cu_seqlens,
                           void* out, float* hT, int B, int T, int H, int S,
                           int D, void* stream, int dtype);

/*
 * gdn_bwd -- gradients of the gated delta rule's forward pass (gdn_fwd's
 * operation) for training: given the output gradient dout and the final-state
 * gradient dhT, it returns the gradients of <dout, out> + <dhT, hT> with
 * respect to q, k, v, g, beta and h0.  The pages train through this layer
 * with a backward pass that recomputes what it needs from the saved inputs
 * ("Optimization Quartet", sections 3.3-3.4; "Model Architecture
 * Walkthrough", section 6.5); so does this one: it takes only the forward's
 * inputs, not its outputs.
 *
 * Arguments and layouts are gdn_fwd's (dense or packed, the same dtype for
 * q, k, v, dout, dq, dk and dv), plus:
 *   dout : like out           dtype     gradient of the output
 *   dhT  : (B, H, dk, dv)     float32   gradient of hT, or NULL (zero)
 *   dq, dk : like q           dtype     written (bf16: round to nearest even)
 *   dv   : like v             dtype     written
 *   dg, dbeta : like g        float32   written
 *   dh0  : (B, H, dk, dv)     float32   written, or NULL (not wanted); it is
 *                                       the gradient of h0 whether or not h0
 *                                       was given
 *   workspace : DEVICE buffer of at least gdn_bwd_workspace_size(...) bytes,
 *        4-byte aligned, owned by the caller; overwritten (no contents needed
 *        on entry or kept on return).  Calls that share a workspace must be
 *        ordered (one stream, or synchronised); overlapping calls race.  It holds, per head and 32-token chunk, two 32x32 fp32
 *        matrices, the state at the chunk's entry and the gradient reaching
 *        its exit state (dk x dv fp32 each): about
 *        (total tokens / 32 + B + 1) * H * (8 KB + 8 dk dv) bytes.
 *
 * Sizes: as for gdn_fwd (dk, dv in {32, 64, 128}; H <= 65535).  Pointers:
 * the inputs and the five token gradients are required when T > 0; the
 * workspace when B > 0.  No output may alias an input or another output.
 *
 * Behaviour: host-side arguments are validated first; on any error a
 * negative status is returned and nothing is launched.  Results are valid
 * once the stream has been synchronised, and bitwise reproducible on one
 * device (no atomics).
 *
 * GDN_BF16 with dk = dv = 128 and a 16-byte-aligned workspace: three
 * kernels with 64-token chunks, every product on the bf16 matrix cores with
 * fp32 accumulation: the forward recurrence saving each chunk's entry state
 * and U, the state gradient swept backwards over the chunks saving each
 * chunk's exit gradient and dX, then the per-chunk token gradients.  The
 * sweeps run as gdn_fwd's sequence segments (cut as there, halos bounded
 * as there; a packed sequence equals the same sequence alone bit for
 * bit).  The saved matrices are bf16, so the gradients carry bf16-level
 * rounding (about 5e-3 of their scale); the workspace use is a prefix of
 * 96 KB per (64-token chunk, head).
 *
 * Other shapes and GDN_F32: four kernels with 32-token chunks (chunk
 * matrices, chunk-entry states, the state gradient swept backwards, the
 * per-chunk token gradients), arithmetic fp32 throughout (bf16 storage is
 * widened on load).  A dense batch with fewer chains x 16-column tiles than twice
 * the device's CUs, and at least 16 chunks per sequence, runs the two
 * sweeps as sequence segments: a segment's state sweep starts from zero at
 * the latest chunk boundary behind it where the product of the per-token
 * transition norms exp(g) max(1, |1 - beta |k|^2|) is below e^-40 (or from
 * h0 at the sequence start), and its gradient sweep from zero at the
 * earliest boundary after it where the product is below that bound (or
 * from dhT at the sequence end); so the result differs from an uncut run
 * by less than that factor beyond rounding.  Packed batches are never cut.
 * The library allocates nothing and keeps no pointer.
 */
int gdn_bwd(const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* h0, const int32_t* cu_seqlens,
            const void* dout, const float* dhT, void* dq, void* dk, void* dv,
            float* dg, float* dbeta, float* dh0, void* workspace,
            long long workspace_bytes, int B, int T, int H, int dk_, int dv_,
            void* stream, int dtype);

/*
 * gdn_fwd_train -- gdn_fwd for training: the same outputs (out and hT equal
 * gdn_fwd's bit for bit, with flags 0), and in the same pass the per-chunk
 * records gdn_bwd's first kernel would otherwise recompute -- each 64-token
 * chunk's entry state and its corrected values U (bf16) -- written into
 * workspace, so that gdn_bwd_saved can skip that kernel.  The pages'
 * fused kernel likewise keeps the forward's states for its backward instead
 * of recomputing them, at the price of extra HBM writes ("Model Architecture
 * Walkthrough", sections 6.5 and 6.8); here one state per 64-token chunk is
 * kept, not one per token.
 *
 * Arguments as gdn_fwd's, without flags, plus workspace / workspace_bytes:
 * a DEVICE buffer of at least gdn_bwd_workspace_size(B, T, H, dk, dv,
 * cu_seqlens != NULL) bytes, 16-byte aligned, owned by the caller; its
 * records stay valid for gdn_bwd_saved on the same inputs until the buffer
 * is written again.  Only the full-width shapes have records: GDN_BF16 with
 * dk = dv = 128 and 64-token chunks (chunk 0 or 64); other valid requests
 * return GDN_ERR_UNSUPPORTED and launch nothing (use gdn_fwd and gdn_bwd).
 * Errors and the rest of the behaviour are gdn_fwd's.
 */
int gdn_fwd_train(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  void* out, float* hT, int B, int T, int H, int dk, int dv,
                  void* stream, int dtype, int chunk, void* workspace,
                  long long workspace_bytes);

/*
 * gdn_bwd_saved -- gdn_bwd for a workspace that already holds the records
 * gdn_fwd_train wrote for the same q, k, v, g, beta, h0 and cu_seqlens (the
 * caller's promise: other inputs give wrong gradients): gdn_bwd without its
 * first kernel.  Arguments, layouts and results are gdn_bwd's; the
 * gradients equal gdn_bwd's bit for bit, except after a gdn_fwd_train call
 * whose hT aliased h0 (its records then come from an uncut recurrence and
 * the gradients differ within rounding).  Only the full-width shapes
 * (GDN_BF16, dk = dv = 128, a 16-byte-aligned workspace) are accepted;
 * other valid requests return GDN_ERR_UNSUPPORTED and launch nothing.
 */
int gdn_bwd_saved(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, const int32_t* cu_seqlens,
                  const void* dout, const float* dhT, void* dq, void* dk, void* dv,
                  float* dg, float* dbeta, float* dh0, void* workspace,
                  long long workspace_bytes, int B, int T, int H, int dk_, int dv_,
                  void* stream, int dtype);

/*
 * gdn_bwd_workspace_size -- bytes of workspace gdn_bwd needs for these sizes
 * (packed != 0: T is the total token count of a packed batch of B
 * sequences).  Returns a negative status for sizes gdn_bwd rejects.
 */
long long gdn_bwd_workspace_size(int B, int T, int H, int dk, int dv,
                                 int packed);

/*
 * gdn_bwd_noalloc -- gdn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, which is instead a
 * fixed scratch array inside the library's device code, one per GPU, of
 * 64 MiB (67108864 bytes), held from the library's first use on that GPU
 * until the process ends.  Its address is looked up once per
 * GPU (hipGetSymbolAddress) on the first call there; no call allocates or
 * frees anything.  Results are those of gdn_bwd on the same inputs.
 *
 * Errors: as gdn_bwd, plus GDN_ERR_SCRATCH when gdn_bwd_workspace_size(...)
 * exceeds 64 MiB (nothing is launched; at dk = dv = 128 and H = 16 that is
 * beyond about 900 tokens), and GDN_ERR_LAUNCH when the
 * scratch address cannot be looked up.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap on one GPU (different streams, or
 * different host threads without ordering) race and give wrong results;
 * order them on one stream.  The scratch needs no contents on entry.
 */
int gdn_bwd_noalloc(const void* q, const void* k, const void* v,
                    const float* g, const float* beta, const float* h0,
                    const int32_t* cu_seqlens, const void* dout,
                    const float* dhT, void* dq, void* dk, void* dv, float* dg,
                    float* dbeta, float* dh0, int B, int T, int H, int dk_,
                    int dv_, void* stream, int dtype);

/* Human-readable text for a status code (static storage, never NULL). */
const char* gdn_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
