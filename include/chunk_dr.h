/*
 * chunk_dr.h -- C interface of the chunked gated delta-rule forward for MI355X (gfx950).
 *
 * The operation (page "PyPTO-Gym 的 chunk_kda 算子实战", sections 算子定位与算法背景
 * and M1-M4): for every sequence n and head h, starting from a K x V state S
 * (the transpose of initial_state[n, h], or zero), and for every token t in order,
 *
 *     S   <- diag(exp(g_t)) S                  per-dimension gate (g_t in R^K), or the
 *                                              scalar per-head gate g_t times the identity
 *     S   <- S + beta_t k_t (v_t - S^T k_t)^T
 *     o_t <- scale * S^T q_t
 *
 * evaluated chunk by chunk (chunk_size tokens; chunks restart at every sequence
 * start): an in-chunk prefix sum of g, the decayed strictly lower-triangular
 * A = beta k k^T, the inverse of (I + A), the w/u projections, and an fp32 state
 * carried from one chunk to the next.  The final state is returned as
 * [N, H, V, K], the transpose of the internal K x V matrix, as on that page
 * (section 算子签名与 I/O 规格).
 *
 * Two variants of the inputs are supported.  Grouped value heads: HV value heads (v, g,
 * beta, o, state) share H query/key heads in groups of HV / H, value head hv reading key
 * head hv / (HV / H), as in the workloads of the page "flash-linear-attention 中的
 * G_T_CONTIG" (H = 4, HV = 8).  In-kernel normalisation (the wrapper switch
 * use_qk_l2norm_in_kernel of the chunk_kda page, section 测试与验证体系): q_t and k_t are
 * replaced by x / sqrt(|x|^2 + 1e-6) over K before anything else.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers to contiguous row-major buffers.
 *  - Tokens are packed: fixed-length batches are addressed as B*T consecutive tokens
 *    (sequence b owns tokens [b*T, (b+1)*T)); a varlen batch has B == 1 and its
 *    sequences are given by cu_seqlens.
 *  - The caller owns every buffer.  The library never allocates, frees, copies
 *    to the host or synchronises; kernels are queued on the given stream and the
 *    call returns immediately.
 *  - Errors are returned as cdr_status values; nothing is printed or thrown.
 */
#ifndef CHUNK_DR_H
#define CHUNK_DR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CDR_VERSION 8

typedef enum {
    CDR_OK = 0,
    CDR_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
    CDR_ERR_BAD_SHAPE = 2,     /* non-positive or inconsistent sizes */
    CDR_ERR_UNSUPPORTED = 3,   /* K or V != 128, chunk_size not 64 or 128, unknown gate */
    CDR_ERR_VARLEN_BATCH = 4,  /* cu_seqlens given with B != 1 */
    CDR_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than cdr_workspace_bytes() */
    CDR_ERR_HIP = 6,           /* a kernel launch failed (hipGetLastError) */
    CDR_ERR_SCRATCH_LIMIT = 7  /* chunk_dr_fwd_noalloc: the problem needs more workspace than its
                                  static array holds (CDR_NOALLOC_SCRATCH_BYTES) */
} cdr_status;

typedef enum {
    CDR_GATE_PER_DIM = 0,      /* g [B*T, HV, K] fp32: per-key-dimension log gate (KDA) */
    CDR_GATE_PER_HEAD = 1      /* g [B*T, HV] fp32: one log gate per token and head (Gated DeltaNet) */
} cdr_gate;

/* Problem description.  All fields are plain host values. */
typedef struct {
    int32_t B;                  /* batch rows; must be 1 when varlen != 0 */
    int32_t T;                  /* tokens per batch row (total packed tokens when varlen) */
    int32_t H;                  /* query/key heads */
    int32_t K;                  /* key dimension; must be 128 */
    int32_t V;                  /* value dimension; must be 128 */
    int32_t N;                  /* sequences: B when varlen == 0, else len(cu_seqlens) - 1 */
    int32_t gate;               /* cdr_gate */
    int32_t chunk_size;         /* 64 or 128 */
    float scale;                /* multiplies q; the usual choice is K^-0.5 */
    int32_t has_initial_state;  /* initial_state is read when non-zero, else S starts at 0 */
    int32_t output_final_state; /* final_state is written when non-zero */
    int32_t varlen;             /* cu_seqlens is read when non-zero */
    int32_t HV;                 /* value heads (v, g, beta, o and the state); 0 means H.  Must be a
                                   multiple of H: value head hv uses query/key head hv / (HV / H) */
    int32_t qk_l2norm;          /* when non-zero, q and k are L2-normalised over K per token inside
                                   the kernels, x / sqrt(|x|^2 + 1e-6) */
} cdr_problem;

/*
 * Host-only validation of a problem description; never touches the device.  The rules are the
 * input checks of the chunk_kda page's host wrapper (section 主机侧 wrapper 与输入校验: K = V =
 * 128, a batch of one with cu_seqlens, shapes that agree), with the page's fixed-length
 * T % 128 == 0 relaxed: any T is accepted, a short last chunk being zero-filled as the page does
 * for varlen tails.  Dtypes are not described here (the interface is untyped); the Python
 * binding checks them.  Returns CDR_OK or the first violated rule (see cdr_status).
 */
cdr_status cdr_check(const cdr_problem* p);

/*
 * Bytes of device workspace chunk_dr_fwd needs for problem p (0 if p is invalid).  The
 * workspace replaces the intermediate tensors of the page's wrapper (section 主机侧 wrapper 与
 * 输入校验 allocates them per call); here the caller owns it.  The size depends only on the
 * shape fields (B, T, H, HV, K, V, N, chunk_size): per chunk and value head the factors of the
 * chunk step (-P split in two bf16 parts, B in fp32, Q, U, exp(gamma_C)) and the chunk-entry
 * state, 224.5 KiB at chunk_size 128 and 192.5 KiB at 64, plus up to 512 per-workgroup scratch
 * slots of 36 KiB (20 KiB at 64).
 */
size_t cdr_workspace_bytes(const cdr_problem* p);

/*
 * Chunked gated delta-rule forward.
 *
 *   q, k          bf16 [B*T, H, K]   queries and keys
 *   v             bf16 [B*T, HV, V]  values (HV value heads, see cdr_problem)
 *   g             fp32 [B*T, HV, K] (CDR_GATE_PER_DIM) or [B*T, HV] (CDR_GATE_PER_HEAD);
 *                 log-domain forget gate.  Supported: every finite g <= 0 (the page's gates
 *                 are logsigmoid values); the in-chunk sums of g must be finite in fp32.
 *                 A key dimension whose gate sums to more than 32 in magnitude over half a
 *                 16-token tile takes, in that tile, pivots that bound every factor by 1 and
 *                 an exact sum over the tile's own pairs (one exponential per pair); the
 *                 other dimensions and tiles are unaffected.  With every dimension that
 *                 strong, the forward takes about 40 % longer than with ordinary gates; with
 *                 a few strong dimensions, about 8 %.  g > 0 is outside the contract (the
 *                 state can then grow without bound).
 *   beta          fp32 [B*T, HV]     delta-rule step size
 *   initial_state fp32 [N, HV, V, K] read when p->has_initial_state, else may be NULL
 *   cu_seqlens    int32 [N + 1]      device array of sequence offsets into the packed token
 *                                    axis (0 = cu[0] <= cu[1] <= ... <= cu[N] = T); read when
 *                                    p->varlen, else may be NULL.  Its contents are not
 *                                    validated; offsets outside [0, T] are undefined behaviour.
 *   o             bf16 [B*T, HV, V]  output, written for every token of every sequence
 *   final_state   fp32 [N, HV, V, K] written when p->output_final_state, else may be NULL.
 *                                    An empty sequence returns its initial state (or zeros).
 *   workspace     device buffer of at least cdr_workspace_bytes(p) bytes, 256-byte aligned;
 *                 its contents on entry do not matter.  It must not be used by another call
 *                 until the kernels of this call have finished on `stream`.
 *   stream        hipStream_t to launch on (NULL = the default stream)
 *
 * The result does not depend on the contents of the workspace or on previous calls:
 * repeated calls on the same inputs give bit-identical o and final_state.
 * Returns CDR_OK after queueing the kernels, or an error status without launching
 * anything (CDR_ERR_HIP if a launch failed).
 */
cdr_status chunk_dr_fwd(const cdr_problem* p,
                        const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const float* initial_state, const int32_t* cu_seqlens,
                        void* o, float* final_state,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device-side check of the contents of cu_seqlens, which chunk_dr_fwd does not read on the
 * host and does not validate.  The rules are the varlen input checks of the chunk_kda page's
 * host wrapper (section 主机侧 wrapper 与输入校验) and of the G_T_CONTIG page's varlen checklist
 * (section 3): the offsets start at 0, never decrease, and end at the total token count.
 *
 *   cu_seqlens  int32 [N + 1] device array
 *   N           sequences, >= 1
 *   T           total packed tokens, >= 0 (the problem's T)
 *   result      device int32, written by the check: 0 when every rule holds, else i + 1 for
 *               the first index i in 0..N where one fails (cu[0] != 0; cu[i] < cu[i - 1];
 *               cu[i] outside 0..T; cu[N] != T)
 *   stream      hipStream_t to launch on (NULL = the default stream)
 *
 * Queues one small kernel and returns without waiting; read *result after the stream has
 * finished it.  The kernel writes *result on every call, so no clearing is needed and the call
 * can be captured in a graph.  Returns CDR_ERR_NULL_ARG for a NULL array or result,
 * CDR_ERR_BAD_SHAPE for N < 1 or T < 0, CDR_ERR_HIP if the launch failed, else CDR_OK.
 */
cdr_status cdr_check_cu_seqlens(const int32_t* cu_seqlens, int32_t N, int32_t T, int32_t* result, void* stream);

/*
 * The same forward, split into its three kernel stages so that each can be timed or
 * profiled on its own.  `stages` is a bit mask of
 *   CDR_STAGE_INTRA  (1)  per-chunk work independent of the carried state: gate prefix sum,
 *                         decayed A and its inverse, w, u (page sections M1-M3), and the
 *                         factors of the chunk step of section M4 re-associated, P = kg^T w,
 *                         B = kg^T u, Q = qg - A2 w, U = A2 u
 *   CDR_STAGE_CHAIN  (2)  the sequential chunk-to-chunk state recurrence
 *                         S <- exp(gamma_C) S - P S + B, the chunk-entry states and the final
 *                         state (section M4; the same sums as u - w S carried through v_new)
 *   CDR_STAGE_OUTPUT (4)  o = Q S_entry + U for every chunk (= qg S + A2 v_new, section M4)
 * Stages run in this order.  A stage reads what earlier stages left in the workspace, so a
 * call with a stage whose predecessors are not in `stages` is only meaningful after a call
 * with the same problem, inputs and workspace that ran them.  chunk_dr_fwd(...) is
 * chunk_dr_fwd_stages(..., CDR_STAGE_ALL, stream).  Arguments and errors as chunk_dr_fwd;
 * a mask outside 1..7 returns CDR_ERR_UNSUPPORTED.
 */
#define CDR_STAGE_INTRA 1
#define CDR_STAGE_CHAIN 2
#define CDR_STAGE_OUTPUT 4
#define CDR_STAGE_ALL 7
cdr_status chunk_dr_fwd_stages(const cdr_problem* p,
                               const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const float* initial_state, const int32_t* cu_seqlens,
                               void* o, float* final_state,
                               void* workspace, size_t workspace_bytes,
                               int32_t stages, void* stream);

/* ------------------------------------------------------------------------------------------
 * The forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * chunk_dr_fwd_noalloc is chunk_dr_fwd (same arguments, same kernels, same bits) with its
 * workspace in a static device array of CDR_NOALLOC_SCRATCH_BYTES owned by the library: one such
 * array per device the entry point runs on, taken when the library's code for it is first used
 * on that device and held until the process ends.  It allocates and frees nothing.  Problems
 * whose cdr_workspace_bytes() exceeds CDR_NOALLOC_SCRATCH_BYTES are rejected with
 * CDR_ERR_SCRATCH_LIMIT before anything is launched; the limit holds the workspace of 8192
 * tokens x 16 heads at chunk_size 128.  The caller still passes (and owns) inputs and outputs.
 *
 * Every call on one device uses that device's one array: two calls whose kernels overlap in time
 * on the same device (different streams, or different threads without ordering) race on it and
 * give undefined results.  Calls ordered on one stream are safe.  The forward reads nothing of
 * the workspace that the same call has not written, so what a previous call left there does not
 * matter and nothing is cleared.
 * ------------------------------------------------------------------------------------------ */
#define CDR_NOALLOC_SCRATCH_BYTES (256u * 1024u * 1024u)
cdr_status chunk_dr_fwd_noalloc(const cdr_problem* p,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const float* initial_state, const int32_t* cu_seqlens,
                                void* o, float* final_state, void* stream);

/* ------------------------------------------------------------------------------------------
 * Context parallelism, the part one device computes (page "flash-linear-attention KCP 精度失效
 * 根因排查手册": a sequence split over ranks, each rank summarising its segment, the summaries
 * exchanged and merged so that each rank learns the state entering its segment).
 *
 * The forward of a segment is affine in its initial state: in the [V, K] layout of the states,
 * final = initial M + X, where X is the final state from a zero start and M ([K, K]) is the
 * product of the segment's chunk maps (exp(gamma_C) - P per chunk, transposed to this layout).
 *
 * chunk_dr_segment_map: M [N, HV, K, K] and X [N, HV, V, K] of every sequence of problem p
 *   (each sequence is one segment).  Arguments as chunk_dr_fwd; p->has_initial_state and
 *   p->output_final_state are ignored.  Uses the forward workspace (cdr_workspace_bytes(p)).
 * chunk_dr_merge_states: given the maps of R consecutive segments of one sequence (M
 *   [R, HV, K, K], X [R, HV, V, K], in order) and the state entering the first (initial_state
 *   [HV, V, K], or NULL for zeros), writes s_in [R + 1, HV, V, K]: s_in[0] = initial_state,
 *   s_in[r + 1] = s_in[r] M[r] + X[r], the state entering segment r + 1; s_in[R] is the final
 *   state.  Running segment r's forward from s_in[r] gives the outputs of the unsplit sequence.
 * On several devices the (M, X) pairs would be all-gathered between the two calls; here they are
 * in one device's memory.
 * ------------------------------------------------------------------------------------------ */
cdr_status chunk_dr_segment_map(const cdr_problem* p,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const int32_t* cu_seqlens,
                                float* M, float* X,
                                void* workspace, size_t workspace_bytes, void* stream);

cdr_status chunk_dr_merge_states(int32_t R, int32_t HV, int32_t K, int32_t V,
                                 const float* M, const float* X, const float* initial_state,
                                 float* s_in, void* stream);

/* ------------------------------------------------------------------------------------------
 * Backward of the chunked forward.
 *
 * The gradients of L = sum(o * do) + sum(final_state * dht) with respect to q, k, v, g, beta and
 * initial_state, for the forward chunk_dr_fwd computes with the same problem p (the vector-
 * Jacobian products of the per-token rule of the chunk_kda page, section 算子定位与算法背景).
 * The backward recomputes what it needs from the inputs (nothing is kept from the forward call):
 * per chunk the decayed blocks, the inverse of (I + A) and the chunk's affine state map, the
 * chunk entry states by a forward chain, the gradients of the chunk exit states by a reverse
 * chain, then all input gradients chunk by chunk.  Storage and the serial chains are fp32; the
 * products run on split-bf16 MFMA (about 16 mantissa bits per operand).
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens  as chunk_dr_fwd
 *   d_o     bf16 [B*T, HV, V]      gradient of o
 *   dht     fp32 [N, HV, V, K]     gradient of the final state, or NULL (zero)
 *   dq, dk  fp32 [B*T, H, K]       written (summed over the value heads of a group)
 *   dv      fp32 [B*T, HV, V]      written
 *   dg      fp32, the shape of g   written
 *   dbeta   fp32 [B*T, HV]         written
 *   dh0     fp32 [N, HV, V, K]     written when p->has_initial_state, else may be NULL
 *   workspace  at least cdr_bwd_workspace_bytes(p) bytes, 256-byte aligned, contents irrelevant
 * Rows of padded or empty chunks are not written; every token of every sequence is.
 * p->output_final_state is ignored.  Errors as chunk_dr_fwd.
 * ------------------------------------------------------------------------------------------ */
size_t cdr_bwd_workspace_bytes(const cdr_problem* p);

cdr_status chunk_dr_bwd(const cdr_problem* p,
                        const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const float* initial_state, const int32_t* cu_seqlens,
                        const void* d_o, const float* dht,
                        float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same backward split into its stages, for timing and profiling.  `stages` is a bit mask of
 *   CDR_BWD_PREP   (1)  per chunk: decayed blocks, (I + A)^-1, w, u, the chunk's state map P, B
 *                       and Q^T do
 *   CDR_BWD_CHAINS (2)  the forward chain (chunk entry states) and the reverse chain (gradients
 *                       of the chunk exit states, dh0)
 *   CDR_BWD_LOCAL  (4)  per chunk: dq, dk, dv, dg, dbeta (and the sum over grouped value heads)
 * Stages run in this order and read what earlier stages left in the workspace, as for
 * chunk_dr_fwd_stages.  chunk_dr_bwd(...) is chunk_dr_bwd_stages(..., CDR_BWD_ALL, stream).
 */
#define CDR_BWD_PREP 1
#define CDR_BWD_CHAINS 2
#define CDR_BWD_LOCAL 4
#define CDR_BWD_ALL 7
cdr_status chunk_dr_bwd_stages(const cdr_problem* p,
                               const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const float* initial_state, const int32_t* cu_seqlens,
                               const void* d_o, const float* dht,
                               float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                               void* workspace, size_t workspace_bytes, int32_t stages, void* stream);

/* ------------------------------------------------------------------------------------------
 * Per-token (recurrent) forward: the decode path.
 *
 * The decode-side companion of the chunked operator (page "PyPTO-Gym 的 chunk_kda 算子实战",
 * section 与其他 KDA 算子的关系): the same update rule as above, applied token by token to an
 * fp32 [HV, V, K] state per sequence, which may be kept in place in a pool of states addressed
 * by slot indices (ssm_state_indices) and may keep one state per draft token for speculative
 * decoding (num_accepted_tokens).  The page names these arguments without defining them; the
 * reading implemented here:
 *
 *  CDR_STATE_SEPARATE  initial_state [N, HV, V, K] (or zeros) in, final_state [N, HV, V, K]
 *                      out, exactly as chunk_dr_fwd.  initial_state and final_state may be the
 *                      same buffer (the update is then in place).
 *  CDR_STATE_POOL      state_pool [num_slots, HV, V, K] fp32, read and written in place;
 *                      ssm_state_indices int32 [N]: sequence n starts from slot idx[n] and its
 *                      state after its last token is written back to slot idx[n].
 *  CDR_STATE_POOL_SPEC ssm_state_indices int32 [N, index_cols]: draft position t of sequence n
 *                      owns slot idx[n, t].  The sequence starts from slot idx[n, a_n - 1], with
 *                      a_n = num_accepted_tokens[n] (int32 [N]; NULL means a_n = 1), and its
 *                      state after its own token t is written to slot idx[n, t] for every
 *                      t < index_cols (later positions have no slot and are not stored).
 *
 * In both pool modes a slot index outside [0, num_slots) marks padding: a start index outside
 * it (or a_n outside 1..index_cols) makes the sequence a padding entry, whose o rows are set to
 * zero and which reads and writes no state; a write index outside it skips that one write.
 * Indices are read on the device and never cause an access outside the pool.  Every start
 * state is read before any state of the same sequence is written, so a sequence may write the
 * slot it starts from; two sequences writing the same slot, or one writing a slot that another
 * starts from, give an undefined result.
 *
 * No workspace: the kernels keep each state row in registers for the whole sequence.
 * ------------------------------------------------------------------------------------------ */
typedef enum {
    CDR_STATE_SEPARATE = 0,
    CDR_STATE_POOL = 1,
    CDR_STATE_POOL_SPEC = 2
} cdr_state_mode;

typedef struct {
    int32_t B;                  /* batch rows; must be 1 when varlen != 0 */
    int32_t T;                  /* tokens per batch row (total packed tokens when varlen) */
    int32_t H;                  /* query/key heads */
    int32_t HV;                 /* value heads, a multiple of H; 0 means H */
    int32_t K;                  /* must be 128 */
    int32_t V;                  /* must be 128 */
    int32_t N;                  /* sequences: B when varlen == 0, else len(cu_seqlens) - 1 */
    int32_t gate;               /* cdr_gate */
    float scale;                /* multiplies q */
    int32_t varlen;             /* cu_seqlens is read when non-zero */
    int32_t qk_l2norm;          /* normalise q and k per token inside the kernel, as chunk_dr_fwd */
    int32_t state_mode;         /* cdr_state_mode */
    int32_t has_initial_state;  /* CDR_STATE_SEPARATE: initial_state is read, else zeros */
    int32_t output_final_state; /* CDR_STATE_SEPARATE: final_state is written */
    int32_t num_slots;          /* pool modes: entries of state_pool (> 0) */
    int32_t index_cols;         /* CDR_STATE_POOL_SPEC: columns of ssm_state_indices (> 0) */
} cdr_recurrent_problem;

/* Host-only validation of a recurrent problem description. */
cdr_status cdr_recurrent_check(const cdr_recurrent_problem* p);

/*
 * Per-token forward.
 *
 *   q, k, v, g, beta, cu_seqlens, o   as chunk_dr_fwd (device pointers, same layouts)
 *   initial_state, final_state        CDR_STATE_SEPARATE only (NULL allowed when the matching
 *                                     flag is 0); ignored in the pool modes
 *   state_pool                        pool modes: fp32 [num_slots, HV, V, K], updated in place
 *   ssm_state_indices                 pool modes: int32 [N] (CDR_STATE_POOL) or
 *                                     [N, index_cols] (CDR_STATE_POOL_SPEC), device
 *   num_accepted_tokens               CDR_STATE_POOL_SPEC: int32 [N], device, or NULL
 *   stream                            hipStream_t (NULL = default stream)
 *
 * One kernel is queued; nothing is allocated, copied to the host or synchronised.  Repeated
 * calls on the same inputs give bit-identical results.  Returns CDR_OK after queueing, or an
 * error status without launching anything (CDR_ERR_HIP if the launch failed).
 */
cdr_status chunk_dr_recurrent_fwd(const cdr_recurrent_problem* p,
                                  const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  const float* initial_state, float* final_state,
                                  float* state_pool, const int32_t* ssm_state_indices,
                                  const int32_t* num_accepted_tokens,
                                  void* o, void* stream);

/* Human-readable name of a status code (static storage). */
const char* cdr_status_str(cdr_status s);

/* CDR_VERSION of the built library. */
int32_t cdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CHUNK_DR_H */
