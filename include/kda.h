/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention chunked-prefill
 * forward library, libkda.so.
 *
 * The operation (named in vLLM PR #55737's report, "Use FlashKDA for KDA
 * chunked prefill", sections "Features and motivation" and "Implementation
 * breakdown", and its FlashKDA wrapper listing under "Key source snippets"):
 * for every sequence n delimited by cu_seqlens and every head h, with
 * head_dim D = 128 and a D x D state S[key c][value j],
 *
 *     q_t, k_t  <- x / sqrt(sum_c x[c]^2 + 1e-6)            (L2 norm in-kernel)
 *     beta_t    =  1 / (1 + exp(-beta_logit_t))              (raw logits in)
 *     log a_t   =  lower_bound * sigmoid(exp(A_log[h]) * (g_t + dt_bias[h]))
 *     S_t       =  (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t       =  scale * S_t^T q_t
 *
 * starting from initial_state (or zeros) and leaving the last S in
 * final_state.  The update and output equations are the plain reading of the
 * gated delta rule the pages name; the gate, the norm, raw beta, the scale on
 * q, the shapes of A_log ([H]) and dt_bias ([H, D]), the workspace query and
 * the fp32 / bf16 checkpoint state follow the wrapper listing and PR #56485's
 * report ("Update flashKDA to support bf16 checkpoint state", "Implementation
 * breakdown").
 *
 * All device pointers are HIP device memory on the current device.  The caller
 * owns every buffer; the library allocates nothing and keeps no state between
 * calls except the test-only overrides below.
 *
 * Status word.  The first 4 bytes of the workspace are an int32 status word.
 * The caller zeroes it once before the workspace's first use (a zero-filled
 * workspace is fine).  The pipelined kernels synchronise their waves through
 * counters with a bounded number of polls; should a wait ever give up (a
 * broken protocol, not an input condition), every wave finishes quickly and a
 * kernel stores a nonzero kind in the status word (1: a wait on the
 * workgroup's LDS counters): the outputs of that call are void.  The library
 * never clears the word, so once the queued work has completed it reports
 * every call made with the workspace since it was last zeroed.  Calls that
 * may run concurrently need workspaces of their own (the sequence order table
 * after the status word is rewritten by calls with more than 16 sequences).
 *
 * Numerics and input range.  Contractions take bf16 operands with fp32
 * accumulation; the state stays fp32 between chunks.  The state update
 * K'^T N takes fp16 operands, N / 16 where N is a chunk's corrected values
 * (N = (I + A)^-1 diag(beta) (V - (e^G k) S)), so |N| must stay below
 * 2^20: values v and state entries up to 2^14 in magnitude are supported
 * (tested against the fp64 recurrence under relative bounds); N overflows to
 * inf, and the state with it, only for inputs of order 2^18 and above.  Below
 * the fp16 range's lower end, N / 16 keeps a relative precision of 2^-11
 * down to 2^-14 and an absolute one of 2^-24 below, i.e. 2^-20 |K'| per term
 * in the update.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
/* Most negative lower_bound the kernels accept: per-token log-decay is in
 * [lower_bound, 0], and the chunk kernel factors exp(G_t - G_i) inside 16-token
 * sub-chunks, whose span must stay inside the fp32 exponent range. */
#define KDA_LOWER_BOUND_MIN (-5.5f)

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1,         /* NULL required pointer, bad size or scalar */
  KDA_ERR_UNSUPPORTED = 2,         /* lower_bound outside [KDA_LOWER_BOUND_MIN, 0] */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < kda_get_workspace_size(...) */
  KDA_ERR_HIP = 4                  /* a HIP launch or device query failed */
} kda_status_t;

typedef enum { KDA_STATE_FP32 = 0, KDA_STATE_BF16 = 1 } kda_state_dtype_t;

/*
 * Bytes of device workspace kda_chunk_prefill_fwd needs for any call with at
 * most max_tokens tokens, heads heads and max_seqs sequences (the query the
 * wrapper listing makes once at construction with max_num_batched_tokens,
 * local_num_heads, max_num_seqs).  Pure, host-only, monotone in every
 * argument.  Returns 0 for negative or zero-sized arguments.
 *
 * The size has two parts.  A call needs the first (the status word and a
 * sequence order table, 4 bytes per sequence); with less it returns
 * KDA_ERR_WORKSPACE_TOO_SMALL.  The second (31.5 MB when max_tokens >= 1024,
 * else none) holds the segment-parallel schedule: long
 * sequences in a call with at most 32 (sequence, head) pairs are cut into
 * segments that run at once (each segment's state map P S + R, then the
 * states entering the segments, then every segment from its state).  A call
 * given only the first part runs every sequence in one piece; results agree
 * within the tolerances, not bit for bit.
 */
size_t kda_get_workspace_size(int64_t max_tokens, int32_t heads, int32_t max_seqs);

/*
 * One KDA chunked-prefill forward over a packed varlen batch.
 *
 *   q, k, v, g     bf16 [num_tokens, heads, 128], dense row-major (device)
 *   beta_logits    bf16 [num_tokens, heads], dense (device); raw logits
 *   A_log          fp32 [heads] (device)
 *   dt_bias        fp32 [heads, 128] (device)
 *   lower_bound    host scalar in [KDA_LOWER_BOUND_MIN, 0]
 *   scale          host scalar (head_dim^-1/2 in the pages), finite
 *   initial_state  [num_seqs, heads, 128, 128] in state_dtype, row index = key
 *                  channel, column = value channel (device); NULL = zeros
 *   cu_seqlens     int32 [num_seqs + 1] (device): cu[0] = 0, non-decreasing,
 *                  cu[num_seqs] <= num_tokens.  Read on the device only; its
 *                  contents are a precondition and are not checked.
 *   out            bf16 [num_tokens, heads, 128] (device); rows of tokens that
 *                  belong to a sequence are written (round to nearest even),
 *                  other rows are not touched
 *   final_state    [num_seqs, heads, 128, 128] in state_dtype (device); may be
 *                  the same pointer as initial_state (in-place update), any
 *                  other overlap is undefined
 *   workspace      device memory of workspace_bytes bytes, at least
 *                  kda_get_workspace_size(num_tokens, heads, num_seqs); its
 *                  first 4 bytes are the status word (zero before the first
 *                  call, see above)
 *   stream         hipStream_t to queue the work on (NULL = default stream)
 *
 * q, k, v, g, beta_logits and out may be NULL when num_tokens is 0; every other
 * pointer except initial_state and workspace is required.  q, k, v, g and out
 * must be 16-byte aligned (the kernels read and write them with 8- and 16-byte
 * accesses).  Size limits:
 * (num_tokens + 256) * heads * 128 < 2^31 (token rows, and rows up to 256
 * past a sequence's end that the kernels read as zeros, are addressed with
 * 32-bit byte offsets), heads <= 65536, num_seqs * heads * 8 < 2^31.
 *
 * Work is queued on the stream and the call returns without waiting: no host
 * synchronisation, no allocation and no device-to-host copy, so the call can be
 * captured into a HIP graph.  All argument checks happen before any HIP call;
 * on an error nothing is launched.  bf16 state is read by exact widening and
 * written once, at the end, rounded to nearest even; the state is fp32 in
 * between.  Results do not depend on the value-dimension split the library
 * picks (bit-identical).
 */
kda_status_t kda_chunk_prefill_fwd(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta_logits, const float* A_log,
                                   const float* dt_bias, float lower_bound, float scale,
                                   const void* initial_state, const int32_t* cu_seqlens, void* out,
                                   void* final_state, void* workspace, void* stream,
                                   int64_t num_tokens, int32_t heads, int32_t num_seqs,
                                   kda_state_dtype_t state_dtype, size_t workspace_bytes);

/*
 * Element strides (counted in elements, not bytes) of the per-token tensors,
 * for kda_chunk_prefill_fwd_strided: row (t, h) of q starts at
 * q + t * q_token + h * q_head and holds its 128 channels contiguously; the
 * same for k, v, g and out; beta_logits[t, h] is at beta + t * beta_token +
 * h * beta_head.  The dense layout of kda_chunk_prefill_fwd is
 * x_token = heads * 128, x_head = 128, beta_token = heads, beta_head = 1.
 */
typedef struct {
  int64_t q_token, q_head;
  int64_t k_token, k_head;
  int64_t v_token, v_head;
  int64_t g_token, g_head;
  int64_t beta_token, beta_head;
  int64_t out_token, out_head;
} kda_strides_t;

/*
 * kda_chunk_prefill_fwd on strided inputs and output, so that a caller whose
 * q, k, v, g are views into a larger projection output (or whose beta logits
 * are a column slice) passes them without dense copies.  The wrapper listing
 * in vLLM PR #55737's report ("Key source snippets") makes such copies because
 * FlashKDA fixes the q/k/v/g strides (only beta may be row-strided); the
 * report's "Risks" list counts their cost.
 *
 *   strides   host pointer (required), see kda_strides_t.  For q, k, v, g and
 *             out, both strides must be non-negative multiples of 8 elements;
 *             beta's strides non-negative.  For each tensor,
 *             (num_tokens + 256) * x_token + (heads - 1) * x_head + 128 < 2^31
 *             (the same 32-bit addressing as the dense call).  Rows of out
 *             that overlap give undefined results.
 *
 * Every other argument, the pointer rules, the limits and the guarantees are
 * those of kda_chunk_prefill_fwd, whose results it reproduces bit for bit for
 * the same values.  q, k, v, g and out must be 16-byte aligned (as in the
 * dense call).
 */
kda_status_t kda_chunk_prefill_fwd_strided(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale,
    const void* initial_state, const int32_t* cu_seqlens, void* out, void* final_state,
    void* workspace, void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype, size_t workspace_bytes, const kda_strides_t* strides);

/*
 * kda_chunk_prefill_fwd (or, with strides, kda_chunk_prefill_fwd_strided) that
 * also writes checkpoint states: the state of each sequence after every
 * `checkpoint_interval` of its tokens.  The PR #56485 report ("Features and
 * motivation") names the kernel's checkpoint state, the intermediate
 * breakpoint used to link a sequence's state across segments, and stores it
 * in the state dtype; the pages give no layout, so this one is the plainest:
 *
 *   checkpoints          device, state dtype (as final_state), laid out
 *                        [checkpoint_capacity, heads, 128, 128] (row = key).
 *                        Sequence n of length L_n writes floor(L_n / interval)
 *                        states; the j-th (j = 1, 2, ..) is the state after
 *                        its first j * interval tokens (computed from
 *                        initial_state like final_state) and goes to slot
 *                        sum_{m < n} floor(L_m / interval) + j - 1.  A
 *                        sequence whose length is a multiple of the interval
 *                        ends with a copy of its final state.  Slots not
 *                        named this way are not written.
 *   checkpoint_interval  tokens between checkpoints, a positive multiple of
 *                        16 (the pipelined kernel's chunk).
 *   checkpoint_capacity  slots in checkpoints: at least
 *                        num_tokens / checkpoint_interval (rounded down),
 *                        which bounds what well-formed cu_seqlens can name;
 *                        slots past the capacity (malformed cu_seqlens) are
 *                        never written.
 *   strides              NULL: the dense layout; else as for
 *                        kda_chunk_prefill_fwd_strided.
 *
 * Every other argument, limit and guarantee is that of the forward call.
 * The work runs on a pipelined kernel whatever the call's size (the 16-token
 * one for lower_bound >= -5, the 32-token one below), always in one piece per
 * sequence (no segment-parallel schedule), so out and final_state are bit for
 * bit those of the forward call given a workspace without the segment area;
 * the forward call differs from them (within the tolerances of the oracle)
 * where it takes the token-serial decode kernel (decode-sized calls, at most
 * 8 tokens per sequence on average) or the segment-parallel schedule.
 * Returns KDA_ERR_INVALID_ARG for a NULL checkpoints, a bad interval or a
 * short capacity, and KDA_ERR_UNSUPPORTED under a kda_debug_set_kernel /
 * kda_debug_set_vsplit override that selects a kernel other than the
 * pipelined ones.
 */
kda_status_t kda_chunk_prefill_fwd_checkpoints(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale,
    const void* initial_state, const int32_t* cu_seqlens, void* out, void* final_state,
    void* workspace, void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype, size_t workspace_bytes, const kda_strides_t* strides,
    void* checkpoints, int32_t checkpoint_interval, int64_t checkpoint_capacity);

/*
 * kda_chunk_prefill_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * allocation): no workspace argument.  The sequence order table, the one
 * scratch buffer of the call (written by a ranking kernel when num_seqs > 16,
 * then read by the forward kernel), lives in a static device array of the
 * library, 65536 entries (256 KiB) per device, held until the process ends;
 * its device address is queried once per device (hipGetSymbolAddress), and the
 * call allocates nothing.
 *
 *   status    device int32 (required): the status word of the workspace
 *             contract (zero it before the first call; nonzero after the work
 *             completes if a kernel gave up a bounded wait).
 *
 * Limits: num_seqs <= 65536 (else KDA_ERR_INVALID_ARG).  Every call on one
 * device shares that device's table, which keeps the last call's contents:
 * calls that may overlap on one device (different streams without ordering
 * between them) race on it and give undefined results.  Every other argument,
 * limit and guarantee is that of kda_chunk_prefill_fwd on dense tensors, with
 * the same results bit for bit as a call given a workspace without the
 * segment area (there is no room for the segment-parallel schedule here, so
 * every sequence runs in one piece).
 */
kda_status_t kda_chunk_prefill_fwd_noalloc(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale,
    const void* initial_state, const int32_t* cu_seqlens, void* out, void* final_state,
    int32_t* status, void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype);

/*
 * One speculative-decode step with num_accepted_tokens rollback.  vLLM PR
 * #55737's report (实现拆解 / "Implementation breakdown" item 4, and the
 * spec-decode discussion under 评论区精华 / "Review highlights") keeps the
 * speculative tokens on a per-token recurrent kernel "with num_accepted_tokens
 * rollback semantics" without defining them; the reading implemented here:
 *
 *   Every sequence n of the step has L_n = cu[n+1] - cu[n] tokens (the
 *   tokens it verifies).  It starts from the state stored after the last
 *   token the previous step accepted: pool slot
 *   state_indices[n][num_accepted_tokens[n] - 1].  It runs the recurrence of
 *   kda_chunk_prefill_fwd over its tokens, writes out as that call does, and
 *   stores the state after its i-th token (i = 0 .. L_n - 1) in pool slot
 *   state_indices[n][i].  Rolling back to an accepted prefix of a tokens is
 *   then the next step's num_accepted_tokens[n] = a: no state is recomputed.
 *
 *   state_pool           device, state dtype, [num_slots, heads, 128, 128]
 *                        (row = key channel, as final_state); read and
 *                        written in place
 *   num_slots            slots in the pool (> 0)
 *   state_indices        device int32 [num_seqs, indices_stride]
 *   indices_stride       slots per sequence (> 0): the most tokens a sequence
 *                        of the step stores a state for
 *   num_accepted_tokens  device int32 [num_seqs]
 *
 * Device-side values are preconditions, not checked: an index outside
 * [0, num_slots), or an accepted count outside [1, indices_stride], makes the
 * sequence start from the zero state (for the start slot) or store nothing
 * (for a token's slot); tokens past indices_stride store nothing.  A slot
 * named by two sequences gives undefined results; the start slot may be
 * among the sequence's own slots (every element is read before it is
 * written).  The work runs on the token-serial decode kernel (4-token
 * staging; the fp32 token-serial kernel under kda_debug_set_kernel(2)), with
 * the arithmetic, the bit-identity across value splits and the other limits
 * and guarantees of kda_chunk_prefill_fwd on dense tensors.  Returns
 * KDA_ERR_INVALID_ARG for a NULL pool, indices or counts, or a non-positive
 * num_slots or indices_stride, and KDA_ERR_UNSUPPORTED under a
 * kda_debug_set_kernel override that selects a chunked kernel.
 */
kda_status_t kda_spec_decode_step(
    const void* q, const void* k, const void* v, const void* g, const void* beta_logits,
    const float* A_log, const float* dt_bias, float lower_bound, float scale, void* state_pool,
    int64_t num_slots, const int32_t* cu_seqlens, const int32_t* state_indices,
    int32_t indices_stride, const int32_t* num_accepted_tokens, void* out, void* workspace,
    void* stream, int64_t num_tokens, int32_t heads, int32_t num_seqs,
    kda_state_dtype_t state_dtype, size_t workspace_bytes);

/*
 * The gate and beta projections upstream of the forward, for few tokens (a
 * decode step): the skinny N and K GEMMs of the PR #55426 report ("Fix KDA
 * projection overlap on Hopper", "Implementation breakdown" items 1-3 and
 * "Key source snippets"), bf16 operands with fp32 accumulation:
 *
 *   P = round_bf16(hidden x w_ab^T)          [num_tokens, n_ab]
 *   G = round_bf16(P[:, :128] x w_b^T)       [num_tokens, n_b]
 *
 * w_ab stacks the gate's first factor (rows 0..127, the rank-128 F_A) over
 * the beta rows (128..n_ab-1); w_b is the gate's second factor (F_B).  The
 * page's test shapes: hidden_dim 7168, n_ab 144, n_b 1536 (12 heads of 128),
 * 2..14 tokens.  G is the forward's raw gate input g [num_tokens, n_b / 128,
 * 128] as it stands, and P's columns 128.. are its raw beta logits: pass them
 * to kda_chunk_prefill_fwd_strided as the column slice P + 128 with
 * beta_token = n_ab, beta_head = 1.  Rounding is to nearest even.  The sum
 * over hidden_dim runs in 1024-wide slices (four 256-wide quarters added in
 * order) whose fp32 partials are added in slice order, so results are
 * run-to-run deterministic.
 *
 *   hidden     device bf16 [num_tokens, hidden_dim], dense
 *   w_ab       device bf16 [n_ab, hidden_dim], dense
 *   w_b        device bf16 [n_b, 128], dense
 *   p_ab, g    device bf16 outputs [num_tokens, n_ab], [num_tokens, n_b]
 *   workspace  device, at least kda_gate_proj_workspace_size(num_tokens,
 *              hidden_dim, n_ab) bytes (partial sums over K slices, written
 *              before they are read: no initialisation needed); calls that
 *              may overlap need workspaces of their own
 *   limits     hidden_dim a positive multiple of 8 (at most 2^24), n_ab a
 *              multiple of 8 in [128, 4096], n_b a positive multiple of 16,
 *              num_tokens in [0, 65536]; hidden, w_ab, w_b, p_ab and the
 *              workspace 16-byte aligned
 *
 * Queued on `stream` (two kernels), no allocation, no host synchronisation.
 * Returns KDA_ERR_INVALID_ARG / KDA_ERR_WORKSPACE_TOO_SMALL before any HIP
 * call, KDA_ERR_HIP if a launch fails.
 */
size_t kda_gate_proj_workspace_size(int32_t num_tokens, int32_t hidden_dim, int32_t n_ab);
kda_status_t kda_gate_proj(const void* hidden, const void* w_ab, const void* w_b, void* p_ab,
                           void* g, void* workspace, size_t workspace_bytes, void* stream,
                           int32_t num_tokens, int32_t hidden_dim, int32_t n_ab, int32_t n_b);

/* Static, human-readable name of a status code (never NULL). */
const char* kda_status_string(kda_status_t status);

/*
 * Detail of the most recent KDA_ERR_HIP returned on the calling thread: the HIP
 * error name and text and the step that failed ("" if there was none).  The
 * string belongs to the library and stays valid until the next call on this
 * thread.
 */
const char* kda_last_hip_error(void);

/*
 * Test hook: force the value-dimension split factor (1, 2, 4 or 8; the value
 * dimension is cut into that many slices, each handled by its own workgroup),
 * or 0 to let the library choose (the pages' rule: split when
 * 2 * heads * sequences <= compute units, PR #52458's report, "Features and
 * motivation").  Process-wide.  Returns the previous setting, or -1 (setting
 * unchanged) for an invalid value.
 */
int kda_debug_set_vsplit(int s);

/*
 * Test hook: the segment-parallel schedule -- 0 (default): automatic (at most
 * 32 (sequence, head) pairs and at least 2048 tokens per sequence on average,
 * or at most 16 pairs and at least 1024 tokens; segments of about 128 / heads
 * per call, at least 256 tokens); 1: never;
 * a multiple of 16 from 16 to 2^24: segments of that many tokens whenever
 * the pipelined 16-token kernel runs the call, heads <= 32 and the segment
 * area holds them ((sequences + num_tokens / len) * heads <= 160).
 * Process-wide.  Returns
 * the previous setting, or -1 (setting unchanged) for an invalid value.
 */
int kda_debug_set_segment(int len);

/*
 * Diagnostic: the segment length the segment-parallel schedule would use for a
 * call of these sizes on the pipelined 16-token kernel with a workspace of
 * kda_get_workspace_size bytes (under the current kda_debug_set_segment
 * setting), or 0 when such a call runs every sequence in one piece.  Host
 * only, no HIP call.
 */
int32_t kda_debug_segment_length(int64_t num_tokens, int32_t heads, int32_t num_seqs);

/*
 * Test hook: choose the kernel family -- 0 (default): automatic.  A call
 * with at most 8 tokens per sequence on average over the whole batch
 * (num_tokens <= 8 * num_seqs: decode-sized) takes the token-serial kernel
 * with 4-token staging, whatever its longest sequence; any other call the
 * pipelined 16-token chunk kernel for lower_bound >= -5, else the pipelined
 * 32-token kernel, both with the value dimension split at least in two, except
 * that the 16-token kernel runs in two workgroups per (sequence, head) (a
 * producer and a consumer of all 128 value columns, bit for bit the same
 * results) for 33 to 96 (sequence, head) pairs, and for 97 to 128 pairs in
 * calls of at most 2^17 (token, head) pairs, when twice the pair count fits
 * on the device's compute units and the workspace holds its second part.
 * The two workgroups of a pair hand the chunks over while both run, so that
 * form needs the compute units the call's grid asks for: on a device whose
 * other compute units are held by kernels that never end, its bounded waits
 * give up (status word 1) instead of completing.  The
 * choice is by the batch's average, so one sequence's result may come from
 * either kernel depending on what it is batched with: both follow the
 * recurrence within the tolerances of the oracle, but they are not bit for
 * bit the same.  1: the 64-token chunk kernel (WY/UT with a blocked forward
 * substitution over the 64x64 triangle); 2: the token-serial fp32 kernel
 * (32-token staging), an independent GPU implementation of the same
 * recurrence used to cross-check the chunked ones; 3: the token-serial kernel
 * with 4-token staging; 4: the pipelined 16-token kernel whatever the call's
 * size (lower_bound < -5 goes to the 32-token kernel, a forced unsplit launch
 * to the 64-token kernel); 5: the pipelined 32-token kernel (chunks of two
 * 16-token halves, each with its own decay reference) whatever the call's
 * size; 6: the 16-token kernel in two workgroups per pair for any pair count
 * that fits (at most 128 pairs and twice the pair count within the compute
 * units; the workspace's second part present; no checkpoints), else as 4.  A
 * kda_debug_set_vsplit override keeps the 16-token kernel in one workgroup per
 * value slice.  Process-wide.  Returns the previous setting, or -1
 * (unchanged) for an invalid value.
 */
int kda_debug_set_kernel(int k);

/*
 * Test hook (host only, no device access): 1 if a call with these sizes,
 * lower_bound >= -5, no checkpoints and a workspace with its second part
 * takes the two-workgroup form of the 16-token kernel on a device with cus
 * compute units under the current kda_debug_* settings, else 0 (also for
 * invalid sizes).
 */
int32_t kda_debug_two_workgroups(int64_t num_tokens, int32_t heads, int32_t num_seqs, int32_t cus);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
