/* libkda: Kimi Delta Attention (KDA) on AMD MI355X (gfx950). C ABI.
 *
 * KDA is the fixed-size-state linear-attention layer of Kimi K3 (the "Sequenz" section of
 * the orkas.ai Kimi K3 architecture page: a running state of fixed size that decays, so
 * newer tokens weigh more). Per (sequence, head) the state S is a dk x dv fp32 matrix,
 * rows indexed by key channel, and each token t does
 *
 *     S <- Diag(exp(g_t)) S;   u = v_t - S^T k_t;   S <- S + beta_t k_t u^T;   o_t = S^T q_t
 *
 * i.e. the incoming state goes through a token-dependent transition before the write,
 * which is why per-device states cannot simply be summed (same page, section
 * "Die Rechnung landet in der Bereitstellungsinfrastruktur").
 *
 * Two calls:
 *   kda_chunk_fwd    - prefill: the whole sequence(s), chunkwise parallel. Chunks are split
 *                      into 16-token tiles whose cumulative log-decay stays in [-80, 0]
 *                      because each step's log-decay is >= -5 (section "Eine Untergrenze,
 *                      die einen GPU-Codepfad beseitigte"), so the diagonal tiles use the
 *                      same dense matrix products as all the others.
 *   kda_decode_step  - one new token per sequence; the state is updated in place and the
 *                      work does not grow with the context (studioglobal.ai Kimi K3 pages,
 *                      "KDA haandterer den vedvarende sekvensbehandling" and "Architektur fuer
 *                      lange Kontexte und guenstigeres Decoding"; orkas.ai infrastructure
 *                      section: the state is updated in place).
 *
 * Conventions shared by every call
 *   - Pointers named q, k, v, g, beta, o, S0, S_T, S, workspace, cu_seqlens are DEVICE
 *     pointers (hipMalloc'ed or torch tensors); argument structs live in host memory.
 *   - The caller allocates and owns every buffer it passes. The library allocates no device
 *     memory; its only device memory is the fixed scratch array of kda_chunk_fwd_noalloc
 *     (below). Its only other global state is a per-thread error string and, per device, the
 *     looked-up address of that array; every call is thread safe except that concurrent
 *     kda_chunk_fwd_noalloc calls on one GPU share the array.
 *   - Sizes whose kernels would need more than 2^32 - 1 work-items in one launch are refused
 *     with KDA_ERR_BAD_SHAPE.
 *   - Every call validates its arguments on the host, before any launch, and returns a
 *     kda_status. On failure nothing has been enqueued and kda_last_error() describes why.
 *   - Work is enqueued on the caller's HIP stream (NULL = the default stream) and the call
 *     returns without synchronising. Launch failures are reported as KDA_ERR_HIP.
 *   - Nothing is printed and no exception crosses the ABI.
 *   - Preconditions not checked by default: g in [-5, 0], beta in [0, 1], q and k rows of
 *     unit L2 norm. With the environment variable KDA_CHECK=1, kda_chunk_fwd, kda_decode_step
 *     and kda_decode_multi first run a device check of g and beta, synchronise the stream and
 *     return KDA_ERR_DECAY_RANGE if any value is outside its range. The check keeps its
 *     counters in the call's output buffer o (overwritten by the call afterwards; o overlaps
 *     no input), so it allocates nothing; kda_decode_multi without o then returns
 *     KDA_ERR_UNSUPPORTED. Nothing is clamped.
 *   - When a call returns an error after enqueueing work (KDA_ERR_HIP, KDA_ERR_DECAY_RANGE),
 *     the contents of its outputs are unspecified.
 *   - Layout: token-major, [B, T, H, d] contiguous (d fastest). States [n_seq, H, dk, dv]
 *     fp32 row-major (key channel rows, value channel columns).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,    /* sizes out of range or inconsistent */
    KDA_ERR_BAD_DTYPE = 3,    /* dtype combination not offered */
    KDA_ERR_UNSUPPORTED = 4,  /* valid request the library does not implement */
    KDA_ERR_DECAY_RANGE = 5,  /* KDA_CHECK=1 found g outside [-5, 0] or beta outside [0, 1] */
    KDA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than kda_chunk_fwd_workspace_bytes() */
    KDA_ERR_HIP = 7,          /* a HIP runtime call or kernel launch failed */
    KDA_ERR_ALIAS = 8         /* an output overlaps an input it must not overlap */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Arguments of kda_chunk_fwd (prefill).
 *
 *   B, T       dense batch: B sequences of T tokens each. With cu_seqlens: B must be 1 and
 *              T is the packed total length. T = 0 is allowed: no token is read or written
 *              (q, k, v, g, beta and o may then be NULL) and S_T receives S0 (zeros if NULL).
 *   H          heads (independent).
 *   dk, dv     key and value head dims, each in {32, 64, 128}.
 *   chunk      chunk length in {16, 32, 64}; a performance knob (results agree across
 *              chunk lengths to rounding). Each chunk is processed as 16-token tiles.
 *   cu_seqlens device int32 [N + 1], token offsets of N packed sequences (0 = cu[0] <= ...
 *              <= cu[N] = T), or NULL for the dense batch. Chunks never straddle a sequence
 *              boundary and each sequence starts from its own S0[n].
 *   N          number of packed sequences (ignored when cu_seqlens is NULL; n_seq = B then).
 *   act_dtype  dtype of q, k, v.   gate_dtype  dtype of g, beta.   out_dtype  dtype of o.
 *              Offered: act = gate = BF16 or act = gate = F32; out F32 or BF16.
 *   q, k, g    [B, T, H, dk];  v [B, T, H, dv];  beta [B, T, H].  Read only.
 *              g is the natural-log per-step decay of each key channel, beta the write
 *              strength.
 *   S0         [n_seq, H, dk, dv] fp32 initial states, or NULL for zeros.
 *   o          [B, T, H, dv] out_dtype. Written. Must not overlap any input.
 *   S_T        [n_seq, H, dk, dv] fp32 final states, or NULL. May be the same buffer as S0
 *              (continue in place); must not partially overlap it.
 *   workspace  device scratch of at least kda_chunk_fwd_workspace_bytes() bytes (may be NULL
 *              when that is 0), 256-byte aligned; contents on entry are ignored.
 *   flags      0, or any of:
 *              KDA_FLAG_GENERIC to force the fp32 vector-ALU path (needs no workspace; slower;
 *              used to cross-check the matrix-core path);
 *              KDA_FLAG_PAIRWISE_DIAG to evaluate the diagonal 16-token tiles of the
 *              matrix-core path pairwise (each e^{G_r - G_j} per pair and key channel, fp32, on
 *              the vector ALUs) as the earlier generation did, instead of by the dense product
 *              that the decay bound makes possible (orkas.ai Kimi K3 page, "Eine Untergrenze, die
 *              einen GPU-Codepfad beseitigte"). It needs no lower bound on g (any g <= 0) and is
 *              slower: the ablation of that bound. (KDA_CHECK=1 still checks g >= -5.)
 *              KDA_FLAG_WALK64 / KDA_FLAG_WALK128 to make the matrix-core path's serial walk
 *              over the chunks take one 64-token chunk per step, or two consecutive chunks
 *              composed into one 128-token step (S -> S + Z + Psi S for the pair, formed in
 *              parallel beforehand). Performance knobs (results agree to rounding): composing
 *              halves the serial steps and the workspace bytes per token, at about 30 % more
 *              parallel work. Without either flag the library composes when there are at most
 *              8 (sequence, head) pairs (where the serial walk dominates). One chunk per step is
 *              always taken when ckpt_every is not a multiple of 128, since checkpoints are
 *              taken between steps (KDA_FLAG_WALK128 is then refused); the workspace size
 *              depends on ckpt_every, so query it with the same value.
 *   ckpt, ckpt_every, ckpt_slots
 *              Sparse state checkpoints for prefix reuse: the fixed-size state is the whole
 *              memory of a prefix, so a later request that shares the prefix can resume from
 *              a stored state instead of recomputing it (orkas.ai Kimi K3 page, the
 *              serving-infrastructure section on per-request state). ckpt_every = 0 writes
 *              none (ckpt and ckpt_slots are then ignored). Otherwise ckpt_every is a positive
 *              multiple of chunk, and ckpt is fp32 [ckpt_slots, H, dk, dv]: checkpoint j >= 1
 *              of sequence n is its state after its first j * ckpt_every tokens (for every j
 *              with j * ckpt_every <= len_n), stored in slot
 *                  sum_{m < n} floor(len_m / ckpt_every) + j - 1.
 *              Slots at or past ckpt_slots are not written (a caller that allocates
 *              sum_n floor(len_n / ckpt_every) slots gets every checkpoint; that sum is at
 *              most floor(B * T / ckpt_every)). ckpt must not overlap any input, o, S_T or
 *              the workspace.
 *   segments   0, 1 or 2: every sequence is walked chunk after chunk (the default). 3 .. 8:
 *              the matrix-core path cuts each sequence into that many segments and walks them
 *              in parallel with the transition form of a segment, S_exit = Phi S_entry + Z
 *              (orkas.ai Kimi K3 page, serving-infrastructure section on splitting a sequence):
 *              one pass computes every middle segment's transition Phi and zero-start summary
 *              Z alongside the first segment, the entries follow in order from those, and a
 *              second pass walks the remaining segments from their entries. It trades about
 *              twice the recurrence work for more parallelism, which pays when few (sequence,
 *              head) pairs leave the GPU idle. The result equals the sequential walk to
 *              rounding; the workspace grows by (3 segments - 5) state-sized buffers. Other
 *              paths ignore it.
 */
typedef struct {
    int B, T, H, dk, dv, chunk;
    const int32_t* cu_seqlens;
    int N;
    kda_dtype act_dtype, gate_dtype, out_dtype;
    const void *q, *k, *v, *g, *beta;
    const float* S0;
    void* o;
    float* S_T;
    void* workspace;
    size_t workspace_bytes;
    unsigned flags;
    float* ckpt;
    int ckpt_every;
    int ckpt_slots;
    int segments;
} kda_chunk_args;

#define KDA_FLAG_GENERIC 1u
#define KDA_FLAG_PAIRWISE_DIAG 2u
#define KDA_FLAG_WALK64 4u
#define KDA_FLAG_WALK128 8u

/* Arguments of kda_decode_step: one token for each of N independent sequences.
 *   q, k, g [N, H, dk];  v [N, H, dv];  beta [N, H]   (act_dtype / gate_dtype as above)
 *   S       [N, H, dk, dv] fp32, read and updated in place.
 *   o       [N, H, dv] out_dtype, the output of the new token (read after the update).
 */
typedef struct {
    int N, H, dk, dv;
    kda_dtype act_dtype, gate_dtype, out_dtype;
    const void *q, *k, *v, *g, *beta;
    float* S;
    void* o;
} kda_decode_args;

/* Arguments of kda_decode_multi: m tokens for each of N independent sequences, evaluated
 * from one read of the state. It serves speculative decoding, which must evaluate draft
 * tokens without committing them and then commit the accepted prefix (orkas.ai Kimi K3
 * page, serving-infrastructure section on speculative decoding and in-place state).
 *   m       tokens per sequence, >= 1.
 *   q, k, g [N, m, H, dk];  v [N, m, H, dv];  beta [N, m, H]: token j of sequence n at [n, j].
 *   S       [N, H, dk, dv] fp32. Token j sees the state after tokens 0..j-1 of its sequence.
 *   o       [N, m, H, dv] out_dtype, every token's output (read after its update); or NULL.
 *   accept  device int32 [N], or NULL. NULL: S is left unchanged (verification). Otherwise
 *           S[n] becomes the state after the first clamp(accept[n], 0, m) tokens (commit;
 *           0 leaves S[n] unchanged). A verify call followed by a commit call with the same
 *           inputs replays the accepted tokens; o of the two calls agree bitwise.
 *   Inputs and accept must not overlap S or o; S and o must not overlap.
 */
typedef struct {
    int N, H, dk, dv, m;
    kda_dtype act_dtype, gate_dtype, out_dtype;
    const void *q, *k, *v, *g, *beta;
    float* S;
    void* o;
    const int32_t* accept;
} kda_decode_multi_args;

/* Bytes of device workspace kda_chunk_fwd needs for these arguments (pointers are not
 * inspected); 0 when the chosen path needs none. Validates shapes and dtypes like
 * kda_chunk_fwd and returns SIZE_MAX (with kda_last_error() set) when they are invalid.
 * The matrix-core path needs one 114,688-byte block per 64-token chunk and head when it walks
 * one chunk per step, or one 163,840-byte block per 128 tokens (two chunks) and head when it
 * composes two per step, plus small tables. */
size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_args* args);

/* Prefill: o and S_T from q, k, v, g, beta and S0, enqueued on hip_stream (hipStream_t). */
kda_status kda_chunk_fwd(const kda_chunk_args* args, void* hip_stream);

/* Prefill without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). Same arguments
 * and results as kda_chunk_fwd, except that workspace and workspace_bytes are ignored: the
 * library's own fixed device scratch of KDA_NOALLOC_SCRATCH_BYTES takes the workspace's place.
 * That scratch is a static array of the library, held by every GPU the library runs on from
 * the first use there until the process ends. Calls whose kda_chunk_fwd_workspace_bytes()
 * exceeds KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_WORKSPACE before anything is enqueued (at
 * most 1,170 (64-token chunk, head) pairs with one chunk per walk step, or 819 (128-token
 * block, head) pairs with composed steps; prefill-4k, 4,096 tokens with 16 heads, fits). No device
 * or host memory is allocated. All calls on one GPU share its scratch, whatever their stream:
 * calls that overlap in time on one GPU race (serialise them, e.g. on one stream). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
kda_status kda_chunk_fwd_noalloc(const kda_chunk_args* args, void* hip_stream);

/* Decode: one step for every (sequence, head); S updated in place, o written. */
kda_status kda_decode_step(const kda_decode_args* args, void* hip_stream);

/* Decode, m tokens per sequence: outputs of all m, and optionally the commit of an accepted
 * prefix into S (see kda_decode_multi_args). With o and accept both NULL nothing is done. */
kda_status kda_decode_multi(const kda_decode_multi_args* args, void* hip_stream);

/* Device check of the preconditions on the gates: counts g values outside [-5, 0] and
 * beta values outside [0, 1] (NaN counts as outside); the floor of -5 is the bound on the
 * per-step log-decay (orkas.ai Kimi K3 page, "Eine Untergrenze, die einen GPU-Codepfad
 * beseitigte"). n_g, n_beta elements; dtype of both is gate_dtype.
 *   counts    caller-owned device scratch of n_counts int64 (n_counts >= 1; up to
 *             KDA_CHECK_COUNTERS of them are used, one per workgroup of the check, so
 *             KDA_CHECK_COUNTERS entries give the most parallel check). Must not overlap g or
 *             beta; its contents on return are unspecified.
 * Synchronises hip_stream; *n_bad receives the count. Allocates nothing. */
#define KDA_CHECK_COUNTERS 1024
kda_status kda_check_gates(const void* g, int64_t n_g, const void* beta, int64_t n_beta,
                           kda_dtype gate_dtype, int64_t* counts, int n_counts,
                           void* hip_stream, int64_t* n_bad);

const char* kda_status_string(kda_status s);
const char* kda_last_error(void);   /* detail of the last failure on this thread */
int kda_abi_version(void);           /* KDA_ABI_VERSION of the built library */

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
