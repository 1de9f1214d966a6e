/*
 * gdr.h -- C ABI of libgdr: the chunked gated delta rule (GDN chunked prefill)
 * forward and backward on AMD Instinct MI355X (gfx950).
 *
 * The operation
 * -------------
 * FlashQLA pages ("flashqla-linear-attention", Core API; "FlashQLA
 * Documentation", forward / backward) define the tensors; the recurrence is
 * the gated delta rule of Gated Delta Networks (Yang, Kautz, Hatamizadeh,
 * 2024).  For every sequence n and value head h (q/k head hq = h / (Hv/Hq),
 * grouped value attention), with a K x V fp32 state S:
 *
 *     S_t = exp(g_t) S_{t-1} + beta_t k_t (v_t - exp(g_t) S_{t-1}^T k_t)^T
 *     o_t = scale * S_t^T q_t
 *
 * computed chunk by chunk (64 tokens) in the WY form: per chunk, gamma is the
 * chunk-local inclusive cumsum of g, A = (I + strict_lower(diag(beta) K K^T o
 * exp(gamma_r - gamma_i)))^{-1} is unit lower triangular, and the state moves
 * from chunk to chunk by S <- e^{gamma_L} S + K^T diag(e^{gamma_L-gamma})
 * A (diag(beta) V - diag(beta e^gamma) K S).
 *
 * Tensor layouts (row-major, contiguous, tokens of all sequences flattened):
 *   q, k          [B, T, Hq, K]           in_dtype
 *   v, o, do, dv  [B, T, Hv, V]           in_dtype
 *   g, dg         [B, T, Hv]              g_dtype (natural-log decay, or the
 *                                         gate's raw input with use_gate)
 *   beta, dbeta   [B, T, Hv]              in_dtype
 *   g_cum         [B, T, Hv]              fp32: chunk-local inclusive cumsum of g
 *   A             [B, T, Hv, 64]          in_dtype: row r of a chunk's inverse
 *                                         at token chunk_start + r; columns past
 *                                         a partial chunk are 0
 *   h             [NC, Hv, K, V]          in_dtype: state at the start of each
 *                                         chunk, chunk c of sequence n at row
 *                                         chunk_offsets[n] + c
 *   states        [N, Hv, K, V]           fp32: initial_state, final_state,
 *                                         dht, dh0
 * With state_v_first != 0 every state tensor (h included) is [.., V, K]
 * instead; the results are then bit-identical transposes of the default.
 * Packed variable-length input (cu_seqlens != NULL) has B == 1 and T the total
 * token count; N = number of sequences.  K and V must be 128.
 *
 * Conventions
 * -----------
 * - The caller owns every buffer and the stream.  The library allocates no
 *   device memory, keeps no pointer after a call returns and never
 *   synchronises: work is enqueued on `stream` (a hipStream_t; NULL = the
 *   null stream) and buffers must stay alive until the stream reaches it.
 * - Outputs are overwritten, never accumulated.  Inputs and outputs must not
 *   alias.  Device pointers must be 16-byte aligned.
 * - Every argument is validated on the host before any HIP call; a failure
 *   returns a status (never aborts) and gdr_last_error() describes it.
 * - Results are deterministic: no floating-point atomics, fixed reduction
 *   orders, and a context-parallel plan that depends only on shapes.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_NULL = 1,      /* a required pointer is NULL */
  GDR_ERR_SHAPE = 2,     /* non-positive or inconsistent sizes */
  GDR_ERR_HEAD_DIM = 3,  /* K != 128 or V != 128 */
  GDR_ERR_DTYPE = 4,     /* q/k/v not bf16/fp16, or g not in_dtype/fp32 */
  GDR_ERR_HEADS = 5,     /* Hq > Hv or Hv % Hq != 0 */
  GDR_ERR_VARLEN = 6,    /* malformed cu_seqlens */
  GDR_ERR_WORKSPACE = 7, /* workspace missing or too small */
  GDR_ERR_DEVICE = 8,    /* no gfx950 device current */
  GDR_ERR_HIP = 9,       /* a HIP launch failed */
  GDR_ERR_ARG = 10       /* another bad argument (scale, chunk size, flags) */
} gdr_status;

typedef enum { GDR_BF16 = 0, GDR_FP16 = 1, GDR_FP32 = 2 } gdr_dtype;

typedef struct {
  int32_t B, T, Hq, Hv, K, V;
  int32_t N;                      /* sequences: B, or len(cu_seqlens) - 1 */
  const int32_t* cu_seqlens_dev;  /* device [N+1] token offsets, or NULL (dense) */
  const int32_t* cu_seqlens_host; /* host copy of the same; used to plan launches
                                     without a device-to-host copy; NULL iff the
                                     device pointer is NULL */
  gdr_dtype in_dtype;             /* q, k, v, beta, do, o, A, h and their grads */
  gdr_dtype g_dtype;              /* raw g and dg: in_dtype or GDR_FP32 */
  float scale;                    /* output scale, usually K^-0.5 */
  int32_t state_v_first;          /* 0: states [.., K, V]; 1: [.., V, K] */
  int32_t cp_segments;            /* intra-GPU context parallelism along T:
                                     0 = automatic plan, 1 = off, s > 1 = split
                                     every sequence into up to s segments */
  int32_t wave_tiles;             /* 16-column state tiles per wave in the scans:
                                     0 = automatic, 1 or 2 */
  int32_t use_qk_l2norm;          /* 1: every kernel scales q and k per (token,
                                     head) to unit length over K before use,
                                     x / sqrt(sum x^2 + 1e-6) in fp32, and the
                                     backward's dq, dk are with respect to the
                                     raw q, k; 0: q and k are used as given.
                                     The option the FLA backend pull request
                                     ("[GDN] Add FlashQLA backend dispatch",
                                     the dispatch's argument list) passes as
                                     use_qk_l2norm_in_kernel. */
  int32_t beta_sigmoid;           /* 1: the beta input is a logit and the
                                     recurrence uses sigmoid(beta); dbeta is with
                                     respect to the logit (the PR page's
                                     use_beta_sigmoid_in_kernel) */
  int32_t neg_eigval;             /* 1: the recurrence uses 2 beta (after the
                                     sigmoid when both are set), so the
                                     transition I - beta k k^T may have a
                                     negative eigenvalue; dbeta is with respect
                                     to the input (the PR page's
                                     allow_neg_eigval) */
  int32_t use_gate;               /* 1: g holds the gate's raw input x and the
                                     recurrence's log decay is, per token and
                                     value head h, computed in fp32:
                                       -exp(gate_A_log[h]) * softplus(x + gate_dt_bias[h])
                                     (the Mamba-2 discretisation that Gated
                                     DeltaNet layers use for their decay; the PR
                                     page's use_gate_in_kernel).  g_cum is the
                                     cumsum of that log decay; the backward
                                     then goes through gdr_chunk_bwd_gate. */
  const float* gate_A_log;        /* device [Hv] fp32: required iff use_gate */
  const float* gate_dt_bias;      /* device [Hv] fp32, or NULL for a zero bias;
                                     NULL unless use_gate */
  int32_t h_packed;               /* 1: gdr_chunk_fwd writes the chunk-start
                                     states h in the packed layout that
                                     gdr_chunk_bwd_states reads (below),
                                     whatever state_v_first says; 0: h is
                                     [NC, Hv, K, V] (or [NC, Hv, V, K] with
                                     state_v_first) */
} gdr_problem;

/* Status name ("GDR_ERR_SHAPE", ...). */
const char* gdr_status_string(gdr_status s);

/* Description of the last failure in the calling thread ("" if none). */
const char* gdr_last_error(void);

/* Host-only argument check, the analogue of the verifier in the FLA backend
 * pull request ("[GDN] Add FlashQLA backend dispatch", Changes and review
 * threads: K != 128, V != 128 and unsupported dtypes are rejected with a
 * reason).  Writes a NUL-terminated reason into `reason` (may be NULL). */
gdr_status gdr_check_supported(const gdr_problem* p, char* reason, size_t reason_len);

/* Device check: the current HIP device is a gfx950.  GDR_ERR_DEVICE if not. */
gdr_status gdr_check_device(void);

/* Bytes of device workspace gdr_chunk_fwd / gdr_chunk_bwd (and
 * gdr_chunk_bwd_gate) / gdr_chunk_bwd_states need for `p` (0 if `p` is
 * invalid).  Depends only on the problem's shapes.  With use_qk_l2norm the
 * forward (h_packed = 1) and the states backward size for both of their
 * forms: given the forward's unit rows they run as problems without the
 * option, whose plans may differ. */
size_t gdr_chunk_fwd_workspace_size(const gdr_problem* p);
size_t gdr_chunk_bwd_workspace_size(const gdr_problem* p);
size_t gdr_chunk_bwd_states_workspace_size(const gdr_problem* p);

/* Forward ("flashqla-linear-attention", Low-Level API; "FlashQLA
 * Documentation", forward pass returning g, A, o, h, final_state).
 *   in : q, k, v, g, beta; initial_state (nullable, fp32 state layout)
 *   out: g_cum, A, o (required); h (nullable: chunk-start states);
 *        final_state (nullable: output_final_state == False)
 *   workspace: device buffer of gdr_chunk_fwd_workspace_size(p) bytes.  With
 *   use_qk_l2norm and h NULL or packed, its tail holds the q and k rows
 *   normalised once (fwd_prep) for the rest of the forward, which then runs
 *   as a problem without the option. */
gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, const float* initial_state,
                         float* g_cum, void* A, void* o, void* h, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Forward that keeps what the backward needs (the pages' autograd
 * integration, "flashqla-linear-attention", Integration with PyTorch
 * Autograd: the forward saves what its backward takes).  gdr_chunk_fwd with
 * p->h_packed = 1, plus:
 *   out: h (required), the packed chunk-start states gdr_chunk_bwd_states
 *        reads
 *        trans: when the plan splits sequences into T-segments, each
 *        segment's state transition T_seg (S_end = T_seg S_start + B_seg),
 *        fp32 [N * Hv][cp_segments][K][K], gdr_chunk_trans_size(p) bytes;
 *        required when that size is nonzero, ignored (may be NULL) when it
 *        is zero; trans_bytes is its size (GDR_ERR_WORKSPACE when smaller).
 *        Entries of the first and last segment of each sequence are never
 *        written or read.  With p->use_qk_l2norm the buffer also keeps,
 *        after the transitions (256-byte aligned), the q and k rows scaled
 *        to unit length (in_dtype, q's layout) and their fp32 1 / |x| per
 *        (token, q head): the forward normalises the rows once, runs the
 *        rest as a problem without the option, and gdr_chunk_bwd_states
 *        given the buffer does the same, mapping dq, dk back through the
 *        normalisation; gdr_chunk_trans_size is then nonzero whatever the
 *        plan.
 * A forward with h_packed = 1 and the backward that takes its states plan
 * together (one segment count for both, gdr_plan_info), so that the
 * backward applies the transposed T_seg instead of forming its own
 * transitions.  Errors: GDR_ERR_ARG when h_packed != 1, GDR_ERR_NULL for a
 * missing h or trans, else as gdr_chunk_fwd. */
size_t gdr_chunk_trans_size(const gdr_problem* p);
gdr_status gdr_chunk_fwd_states(const gdr_problem* p, const void* q, const void* k,
                                const void* v, const void* g, const void* beta,
                                const float* initial_state, float* g_cum, void* A, void* o,
                                void* h, float* trans, size_t trans_bytes, float* final_state,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Forward without allocation, for callers that cannot call hipMalloc or take
 * a caller-owned workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results and
 * errors as gdr_chunk_fwd (bit-identical outputs: same plan, same kernels),
 * with no workspace: the library uses a static device array of 64 MiB per
 * GPU (GDR_NOALLOC_SCRATCH_BYTES), allocated when the library's code object
 * loads on that GPU and held until the process ends.  Problems whose
 * gdr_chunk_fwd_workspace_size exceeds it are rejected with
 * GDR_ERR_WORKSPACE before any device work (a single 65,536-token sequence
 * with 32 value heads needs 48 MiB; short and dense problems need none).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several threads) race and must not be
 * issued.  Nothing in the array needs to start at zero: each call writes
 * every byte it later reads. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k,
                                 const void* v, const void* g, const void* beta,
                                 const float* initial_state, float* g_cum, void* A, void* o,
                                 void* h, float* final_state, void* stream);

/* Backward ("FlashQLA Documentation", backward pass: takes q, k, v, the g
 * returned by the forward, beta, A, do, dht, scale, initial_state, cu_seqlens
 * and returns dq, dk, dv, db, dg, dh0).
 *   in : q, k, v, g_cum (the forward's fp32 g output), beta, A (forward
 *        output), do; dht (nullable = zero); initial_state (nullable = zero)
 *   out: dq, dk (in_dtype, [B,T,Hq,K]); dv; dbeta; dg (g_dtype, gradient with
 *        respect to the raw g); dh0 (fp32, written iff initial_state != NULL,
 *        may be NULL otherwise)
 *   Problems with use_gate are rejected (GDR_ERR_ARG): see gdr_chunk_bwd_gate.
 *   workspace: device buffer of gdr_chunk_bwd_workspace_size(p) bytes. */
gdr_status gdr_chunk_bwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* g_cum, const void* beta, const void* A, const void* do_,
                         const float* dht, const float* initial_state, void* dq, void* dk,
                         void* dv, void* dbeta, void* dg, float* dh0, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Backward with the in-kernel gate (problem->use_gate == 1; gdr_chunk_bwd
 * rejects such problems).  The arguments of gdr_chunk_bwd, plus:
 *   in : g, the gate's raw input x the forward took (g_dtype [B,T,Hv])
 *   out: dg is the gradient with respect to x (g_dtype);
 *        dA_log, ddt_bias (fp32 [Hv], each nullable = not written): the
 *        gradients of gate_A_log and gate_dt_bias, sums over every token of
 *        every sequence, in a fixed order (deterministic)
 * The workspace (gdr_chunk_bwd_workspace_size) includes 8 bytes per chunk
 * and value head for the per-chunk partial sums of those two gradients. */
gdr_status gdr_chunk_bwd_gate(const gdr_problem* p, const void* q, const void* k, const void* v,
                              const float* g_cum, const void* g, const void* beta, const void* A,
                              const void* do_, const float* dht, const float* initial_state,
                              void* dq, void* dk, void* dv, void* dbeta, void* dg, float* dh0,
                              float* dA_log, float* ddt_bias, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Backward given the forward's chunk-start states: the backward the pages'
 * autograd integration ("flashqla-linear-attention", Integration with
 * PyTorch Autograd) runs after a forward that kept its states.  The
 * arguments and results of gdr_chunk_bwd (gdr_chunk_bwd_gate when
 * p->use_gate), plus:
 *   in : h, the chunk-start states gdr_chunk_fwd computed for the same
 *        problem and inputs with h_packed = 1: per chunk row and value head
 *        the 128 x 128 state in in_dtype as [V/16][K/32][64][8]: element
 *        ((vb * 4 + kb) * 64 + 16 * g + c) * 8 + e holds the state at value
 *        16 vb + c and key 32 kb + 4 g + e (e < 4), 32 kb + 16 + 4 g + e - 4
 *        (e >= 4) -- the order the kernels hold it in, so that it is written
 *        and read in 1 KiB contiguous pieces
 *        trans (nullable), the segment transitions gdr_chunk_fwd_states
 *        kept for the same problem and inputs, trans_bytes its size
 *        (GDR_ERR_WORKSPACE when below gdr_chunk_trans_size); when the plan
 *        splits sequences the state-gradient scan then applies them
 *        transposed (the gradient's transition over a segment is T_seg^T)
 *        instead of forming its own, which halves its transition pass;
 *        NULL: it forms them (ignored when the plan splits nothing).
 *        With p->use_qk_l2norm the buffer's unit rows are used instead of
 *        normalising q and k again (q and k are then not read); NULL: the
 *        backward normalises them itself
 *        g, the gate's raw input (use_gate only; NULL otherwise, and so are
 *        dA_log, ddt_bias)
 * The states are not recomputed: only the reverse state-gradient scan runs
 * before the per-chunk gradients, and the workspace
 * (gdr_chunk_bwd_states_workspace_size) holds no state buffer.  States or
 * transitions from another problem or other inputs give meaningless
 * gradients. */
gdr_status gdr_chunk_bwd_states(const gdr_problem* p, const void* q, const void* k,
                                const void* v, const float* g_cum, const void* g,
                                const void* beta, const void* A, const void* do_,
                                const float* dht, const float* initial_state, const void* h,
                                const float* trans, size_t trans_bytes, void* dq, void* dk,
                                void* dv, void* dbeta, void* dg, float* dh0, float* dA_log,
                                float* ddt_bias, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Token-by-token forward for short inputs: decode steps, a few speculative
 * tokens, or a prefill continued from a cached state (the "state-cached
 * continuation" the "flashqla-linear-attention" page lists among its
 * topics).  The same o and final_state as gdr_chunk_fwd, from the same
 * recurrence, but one token at a time with the fp32 state of each
 * (sequence, value head) held on chip: the state is read once and written
 * once, so a step costs about two state transfers (128 KiB per head).
 *   in : q, k [B,T,Hq,K]; v [B,T,Hv,V]; g (raw log decay, g_dtype) and beta
 *        [B,T,Hv]; initial_state fp32 [N,Hv,K,V] ([N,Hv,V,K] with
 *        state_v_first), nullable = zeros
 *   out: o [B,T,Hv,V] in in_dtype; final_state fp32, same layout as
 *        initial_state, nullable.  final_state may be the same buffer as
 *        initial_state (the state is updated in place); no other argument
 *        may alias another.
 * Honours cu_seqlens, state_v_first, scale, use_qk_l2norm, the beta options
 * and use_gate (g is then the gate's raw input).  Needs no
 * workspace.  Costs grow linearly with T; past a few chunks gdr_chunk_fwd is
 * faster.  Errors as gdr_chunk_fwd (validation on the host first). */
gdr_status gdr_recurrent_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, const float* initial_state,
                             void* o, float* final_state, void* stream);

/* Variable-length helpers (host, pure integer, bit-exact), after the
 * utilities of the "FlashQLA Documentation" page.  `cu` holds n_plus_1
 * non-decreasing offsets starting at 0.  Each returns GDR_ERR_VARLEN for a
 * malformed `cu`, GDR_ERR_ARG for chunk_size < 1.
 *
 * prepare_lens: lens[i] = cu[i+1] - cu[i]   (n_plus_1 - 1 entries). */
gdr_status gdr_prepare_lens_i32(const int32_t* cu, int64_t n_plus_1, int32_t* lens);
gdr_status gdr_prepare_lens_i64(const int64_t* cu, int64_t n_plus_1, int64_t* lens);

/* prepare_chunk_indices: one row per chunk, in sequence order, holding
 * [sequence index n, chunk index j within sequence n]; the chunk's first
 * token is cu[n] + j * chunk_size.  `out` ([num_chunks, 2]) may be NULL to
 * query *num_chunks only. */
gdr_status gdr_prepare_chunk_indices_i32(const int32_t* cu, int64_t n_plus_1, int64_t chunk_size,
                                         int32_t* out, int64_t* num_chunks);
gdr_status gdr_prepare_chunk_indices_i64(const int64_t* cu, int64_t n_plus_1, int64_t chunk_size,
                                         int64_t* out, int64_t* num_chunks);

/* prepare_chunk_offsets: offsets[0] = 0, offsets[i+1] = offsets[i] +
 * ceil(lens[i] / chunk_size) (n_plus_1 entries, the shape of cu), and
 * *total = offsets[n_plus_1 - 1]: the row of chunk c of sequence n in a
 * global per-chunk buffer such as h is offsets[n] + c. */
gdr_status gdr_prepare_chunk_offsets_i32(const int32_t* cu, int64_t n_plus_1, int64_t chunk_size,
                                         int32_t* offsets, int64_t* total);
gdr_status gdr_prepare_chunk_offsets_i64(const int64_t* cu, int64_t n_plus_1, int64_t chunk_size,
                                         int64_t* offsets, int64_t* total);

/* The literal reading of the chunk-index description: one row per chunk
 * holding [first token of the chunk, global chunk id]. */
gdr_status gdr_prepare_chunk_token_starts_i64(const int64_t* cu, int64_t n_plus_1,
                                              int64_t chunk_size, int64_t* out,
                                              int64_t* num_chunks);

/* The launch plan the library picks for `p` in one direction (backward != 0:
 * gdr_chunk_bwd, or gdr_chunk_bwd_states when p->h_packed; else
 * gdr_chunk_fwd / gdr_chunk_fwd_states); it depends only on shapes and those
 * flags.  With p->h_packed both directions share one segment count:
 * *cp_segments = T-segments per sequence (1 = no context parallelism),
 * *wave_tiles = 16-column state tiles per wave in the scans (1 or 2).
 * A nonzero cp_segments / wave_tiles in `p` fixes that choice for both. */
gdr_status gdr_plan_info(const gdr_problem* p, int backward, int32_t* cp_segments,
                         int32_t* wave_tiles);

/* The pipelined backward gdr_chunk_bwd_states runs for `p` (a diagnostic;
 * shapes only).  With at most 128 (sequence, head) units of a dense batch,
 * or 256 of packed sequences without grouped heads, and 16 or more chunks
 * in the longest sequence: *slices = 1: one launch holds the state-gradient
 * scan and the gradient workgroups of every chunk, the chunks nearest their
 * sequence's end first, each starting once the scan has stored its chunk's
 * state gradient (bounds = 0, chunks of the longest sequence).  With
 * use_qk_l2norm (reported for the backward that normalises q and k itself;
 * given the forward's unit rows it runs as without the option), at most 64
 * units of a dense batch and no grouped heads, *slices >= 2: the scan runs in ranges of
 * chunks, the last range first, each launch pairing one range's scan with
 * the per-chunk gradients of the range the launch before finished; the last
 * launch runs the gradients of chunks [bounds[0], bounds[1]) of every
 * sequence alone.  *slices = 0: one scan launch, then one gradient launch.
 * bounds (nullable) receives up to max_bounds of the *slices + 1 range
 * starts (bounds[*slices] = chunks per sequence). */
gdr_status gdr_bwd_pipeline_info(const gdr_problem* p, int32_t* slices, int32_t* bounds,
                                 int32_t max_bounds);

/* Kernel timing for benchmarks and diagnostics (not part of the pages' API).
 * While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events recorded on its stream.  gdr_profile_enable clears the records
 * (and creates events lazily afterwards); gdr_profile_read waits for the
 * recorded events, adds up the elapsed time per kernel name (names such as
 * "fwd_prep", "scan_out", "scan_aug", "scan_state", "cp_combine",
 * "dh_scan_out", "dh_scan_aug", "grad", "gva_reduce", "chunk_offsets"),
 * writes up to max_entries of them (names: NUL-terminated, name_stride bytes
 * apart; total_ms; launches -- each may be NULL), clears the records and
 * returns the number of entries written. */
gdr_status gdr_profile_enable(int enable);
int gdr_profile_read(char* names, size_t name_stride, double* total_ms, int* launches,
                     int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
