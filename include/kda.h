/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) Kimi Delta Attention mixer core.
 *
 * The operation (nnterp Kimi-Linear encyclopedia page, Notes, section on KDA decaying
 * each key channel, and the family-module docstring of section 04): per head, a state
 * S of [key_dim, value_dim] is carried across tokens.  Each token
 *     1. L2-normalises its key and query (the kernel applies the norm) and scales the
 *        query by 1/sqrt(key_dim),
 *     2. decays every key channel i of S by exp(g[i])   (g: natural-log decay, <= 0),
 *     3. applies the delta rule  S += beta * k (v - S^T k)^T,
 *     4. reads  o = S^T q  from the updated state.
 * The kernels take (query, key, value, g=, beta=, initial_state=) and return the head
 * outputs and the last state; initial_state is absent at the start of a prompt
 * (same page, section 02, state_input / state_output rows).  The head outputs then
 * pass a sigmoid-gated RMSNorm with one [head_dim] weight (Kimi-K3 atlas,
 * gate-project page: o_norm code and Parameters table).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers to contiguous row-major buffers owned by
 *    the caller; the library never allocates, frees or retains device memory and keeps
 *    no state between calls (calls are thread-safe).  Scratch space, where a kernel
 *    needs it, is a caller-provided workspace whose size the library reports.
 *    Pointers to tensors with a feature axis (q, k, v, g, states, o, gate, y, weights) must be 16-byte aligned;
 *    beta and cu_seqlens need 4-byte alignment, mask none.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default
 *    stream).  Arguments are validated on the host before anything is launched; a
 *    non-OK status other than KDA_ERR_HIP means nothing was enqueued and no output was
 *    touched (KDA_ERR_HIP: a launch failed, and earlier launches of the same call may
 *    have been enqueued).  Faults inside a kernel surface at the caller's next
 *    synchronisation.
 *  - dtype codes: KDA_F32 = IEEE fp32, KDA_BF16 = bfloat16 (outputs rounded to
 *    nearest-even).  The recurrent state is always fp32.
 *  - Precondition (not checked, documented): every g lies in [-5, 0], the decay lower
 *    bound of the Kimi-K3 configuration (Kimi-K3 atlas, config.json,
 *    linear_attn_config.gate_lower_bound).  The bf16 chunked kernel factors
 *    within-chunk decays with 16-token reference points and stays finite for
 *    g >= -5.4; the other kernels accept any g <= 0.
 *  - Precondition of the bf16 chunked kernel for dk = dv = 128 (not checked,
 *    documented): its state-side matrix-core products take fp16 operands (largest
 *    finite value 65504).  Every |v| entry, and the Euclidean norm of every value column
 *    S[:, j] of the initial state and of every state the sequence reaches, must stay
 *    at or below 2^14 = 16384; the operands (S, v - k^T S and the corrected values) then
 *    stay below 2^15.  Outside that range this kernel may return inf or NaN where the
 *    fp32 token-by-token kernels stay finite.  With unit keys, beta in (0, 1) and g <= 0
 *    a state's column norms grow by at most |beta (v - k^T S)| per token.
 *  - Padded tokens (mask == 0), and tokens of a packed batch, must hold finite values.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,         /* a required pointer is NULL                                   */
  KDA_ERR_SHAPE = 2,        /* a size is out of range or inconsistent                       */
  KDA_ERR_DTYPE = 3,        /* unknown dtype code                                           */
  KDA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned                             */
  KDA_ERR_CONFLICT = 5,     /* mutually exclusive arguments given together                  */
  KDA_ERR_WORKSPACE = 6,    /* the workspace is missing or smaller than required            */
  KDA_ERR_UNSUPPORTED = 7,  /* a valid combination this build has no kernel for             */
  KDA_ERR_HIP = 8,          /* the HIP runtime reported an error at launch                  */
  KDA_ERR_TIMEOUT = 9       /* a bounded wait inside a kernel ran out (kda_chunk_prefill_status) */
} kda_status_t;

/* Problem description shared by the prefill and recurrent entry points. */
typedef struct {
  int32_t B;             /* batch rows; 1 when cu_seqlens packs the sequences              */
  int32_t T;             /* tokens per row (packed total with cu_seqlens)                  */
  int32_t H;             /* heads                                                          */
  int32_t dk;            /* key_dim   (16, 32, 64 or 128)                                  */
  int32_t dv;            /* value_dim (== dk in this build)                                */
  int32_t num_seqs;      /* sequences: len(cu_seqlens)-1 with cu_seqlens, else ignored (=B) */
  int32_t chunk;         /* prefill chunk length: 0 = kernel's choice; 64 or 32 (bf16, d = 128:
                            the matrix-core kernel, whose blocks are 32 tokens; a 64-token
                            chunk is carried as its two halves, the same chunked form
                            regrouped) or 16 (the vector-ALU kernel, any dtype).  The result
                            does not depend on it beyond rounding.                          */
  float scale;           /* query scale; 0 = 1/sqrt(dk)                                    */
  int32_t use_qk_l2norm; /* 1: q, k are L2-normalised in the kernel (x / sqrt(sum x^2 + 1e-6)) */
  int32_t in_dtype;      /* kda_dtype_t of q, k, v and gate                                */
  int32_t out_dtype;     /* kda_dtype_t of o and y                                         */
  float norm_eps;        /* gated-RMSNorm epsilon                                          */
  int32_t decay_per_head; /* 0: g is [B, T, H, dk], one log decay per key channel (KDA);
                            1: g is [B, T, H], one per head, shared by its key channels
                            (the gated DeltaNet's scalar decay; nnterp Kimi-Linear page,
                            Notes: KDA is the gated DeltaNet with the decay made per channel) */
} kda_params_t;

/*
 * kda_chunk_prefill -- the prompt kernel: runs the recurrence over whole sequences,
 * carrying the state from one chunk of tokens to the next without storing it per token
 * (nnterp Kimi-Linear page, Notes, "Loading", which names 64-token chunks; the chunked
 * form is exact for any chunk length; these kernels work in blocks of 32 or 16).  Results equal
 * the token-by-token recurrence up to rounding.
 *
 *   q, k          [B, T, H, dk]   in_dtype
 *   v             [B, T, H, dv]   in_dtype
 *   g             [B, T, H, dk]   fp32 log decays (<= 0); [B, T, H] with p->decay_per_head
 *   beta          [B, T, H]       fp32 write strengths in (0, 1), already sigmoided
 *   initial_state [N, H, dk, dv]  fp32, or NULL for a zero state (start of a prompt)
 *   cu_seqlens    [N + 1]         int32 device array of packed sequence offsets
 *                                 (cu_seqlens[0] = 0, non-decreasing, last <= T), or NULL;
 *                                 requires B == 1 and p->num_seqs = N
 *   mask          [B, T]          uint8, 1 = token, 0 = padding (skipped: state unchanged,
 *                                 output 0), or NULL; not together with cu_seqlens
 *   o             [B, T, H, dv]   out_dtype head outputs (before the gated norm); may be
 *                                 NULL when y is given (only y is then written)
 *   final_state   [N, H, dk, dv]  fp32; may be the same buffer as initial_state
 *   gate          [B, T, H, dv]   in_dtype, norm_weight [dv] fp32, y [B, T, H, dv]
 *                                 out_dtype: the gated norm y = w * o / rms(o) *
 *                                 sigmoid(gate) per head; all three set or all NULL
 *   workspace     device scratch of at least kda_chunk_prefill_workspace_size(p,
 *                 cu_seqlens != NULL) bytes, 16-byte aligned; may be NULL when that size
 *                 is 0.  Its contents on entry do not matter; they are overwritten.
 *                 Calls that overlap in time must not share a workspace.
 * N = B without cu_seqlens.  Tokens of a packed batch outside [0, cu_seqlens[N]) are
 * not written.
 *
 * The bf16 kernel for dk = dv = 128 runs in two launches: a preparation pass over every
 * (sequence, head, chunk) at once, which stores each chunk's intra-chunk products in the
 * workspace (32,272 bytes per chunk and head, plus 512 bytes that kda_chunk_scan's own
 * norm uses), then the sequential state scan; with y and o given, a third launch applies
 * the gated norm to o.  With y given and o NULL the scan writes the head outputs into y
 * and the norm runs on them in place (no work-group of this call waits for another).
 * The vector-ALU kernel applies the norm in its own launch either way.
 */
kda_status_t kda_chunk_prefill(const kda_params_t *p,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const float *initial_state,
                               const int32_t *cu_seqlens, const uint8_t *mask,
                               void *o, float *final_state,
                               const void *gate, const float *norm_weight, void *y,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_prefill_workspace_size -- bytes of workspace kda_chunk_prefill needs for
 * these params; `packed` is nonzero when cu_seqlens will be given (p->num_seqs set).
 * 0 for invalid params or when the chosen kernel needs none.  With packing it is
 * (N + ceil(T / 32)) * H * 32784 + 256 bytes, otherwise B * ceil(T / 32) * H * 32784 + 256
 * (a record and the norm-exchange words per chunk and head, then a status word).
 */
size_t kda_chunk_prefill_workspace_size(const kda_params_t *p, int32_t packed);

/*
 * kda_chunk_prefill_status -- whether every wait between the two column tiles of a head
 * in the scans run on this workspace since its last preparation completed normally.
 * Only the scan that applies the gated norm itself (kda_chunk_scan with y) has such
 * waits: the two work-groups of a head
 * exchange per-token sums of squares.  A wait always ends, since partner work-groups
 * are consecutive in one XCD's dispatch order, but it is bounded (seconds); if other work
 * held the GPU's CUs longer than that, the wait gives up, the tokens after it get NaN in
 * y, and the workspace's status word is set.  This call waits for `stream`, reads that
 * word, and returns KDA_OK or KDA_ERR_TIMEOUT.  p and packed as for
 * kda_chunk_prefill_workspace_size; workspace as given to the prefill.  Errors:
 * KDA_ERR_NULL, KDA_ERR_WORKSPACE, KDA_ERR_UNSUPPORTED (p does not select the
 * matrix-core kernel), KDA_ERR_HIP.  Nothing is allocated; it synchronises the stream.
 */
kda_status_t kda_chunk_prefill_status(const kda_params_t *p, int32_t packed, const void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * kda_chunk_prepare, kda_chunk_scan -- the two launches of kda_chunk_prefill's bf16,
 * dk = dv = 128 kernel, callable one at a time (same chunked form as kda_chunk_prefill;
 * nnterp Kimi-Linear page, Notes, "Loading").  kda_chunk_prefill is exactly
 * kda_chunk_prepare followed by kda_chunk_scan on the same stream (then, with y, the
 * gated norm over o, as kda_gated_rmsnorm).
 *
 * kda_chunk_prepare reads q, k, g, beta (and cu_seqlens or mask, as in kda_chunk_prefill)
 * and fills the workspace with one record per (sequence, head, chunk): everything about a
 * chunk that does not depend on the incoming state.  It needs no state, so it may run
 * ahead of the scan that consumes it.
 *
 * kda_chunk_scan reads v, initial_state (or NULL) and the records, and writes o and
 * final_state (o may be NULL when y is given); with gate, norm_weight and y (all set or
 * all NULL, as in
 * kda_chunk_prefill; eps is p->norm_eps) it also writes the gated norm y itself, in
 * the same launch: each head's 128 value columns are scanned by two work-groups of 64,
 * which exchange per-token sums of squares through the workspace (device-coherent
 * 64-bit words; a wait for the other work-group is bounded and, if it ever ran out,
 * would give NaN in y rather than hang).  That saves the second read of o but loads the
 * scan, so at large T it is slower than writing o and running the separate norm, which
 * kda_chunk_prefill uses.  p and cu_seqlens must be those the workspace was prepared with, and the
 * preparation must have completed or be ordered before the scan on the stream; the
 * workspace must not be modified in between.  The records already hold the effect of a
 * mask, so the scan takes none.
 *
 * Arguments have the meaning, layout and alignment given for kda_chunk_prefill; the
 * workspace is at least kda_chunk_prefill_workspace_size(p, cu_seqlens != NULL) bytes.
 * Both return KDA_ERR_UNSUPPORTED unless p selects the bf16, dk = dv = 128 kernel
 * (in_dtype bf16, chunk 0, 32 or 64, T * H * 128 < 2^31).  Ownership: all buffers stay the
 * caller's; nothing is allocated.  Errors: as for kda_chunk_prefill.
 */
kda_status_t kda_chunk_prepare(const kda_params_t *p,
                               const void *q, const void *k,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens, const uint8_t *mask,
                               void *workspace, size_t workspace_bytes, void *stream);
kda_status_t kda_chunk_scan(const kda_params_t *p, const void *v,
                            const float *initial_state, const int32_t *cu_seqlens,
                            const void *workspace, size_t workspace_bytes,
                            void *o, float *final_state,
                            const void *gate, const float *norm_weight, void *y, void *stream);

/*
 * kda_recurrent_step -- the decode kernel: the token-by-token form, for one new token
 * per row (T = 1) or a few tokens (T >= 1, applied in order).  The state is read and
 * written in place: state [B, H, dk, dv] fp32 holds S before the call and S after the
 * last token on return.  Other arguments as for kda_chunk_prefill (no cu_seqlens), except
 * that o is always required (with few slabs and several tokens the gated norm runs as its
 * own pass over o): NULL o is KDA_ERR_NULL.
 */
kda_status_t kda_recurrent_step(const kda_params_t *p,
                                const void *q, const void *k, const void *v,
                                const float *g, const float *beta,
                                float *state, const uint8_t *mask,
                                void *o,
                                const void *gate, const float *norm_weight, void *y,
                                void *stream);

/*
 * kda_recurrent_states -- kda_recurrent_step that also stores the state after every
 * token: the per-token states a prompt yields when it runs through the token-by-token
 * kernel rather than the chunked one (nnterp Kimi-Linear page, support() table, the
 * 'states' row [batch, seq, heads, key_dim, value_dim]; Notes, "Loading").
 *   states [B, T, H, dk, dv] fp32, 16-byte aligned: states[b, t, h] is S after token t
 *          (for a padding token, the carried state).  64 KB per token and head at d = 128.
 * Other arguments, ownership and errors as for kda_recurrent_step (KDA_ERR_NULL when
 * states is NULL).
 */
kda_status_t kda_recurrent_states(const kda_params_t *p,
                                  const void *q, const void *k, const void *v,
                                  const float *g, const float *beta,
                                  float *state, const uint8_t *mask,
                                  void *o,
                                  const void *gate, const float *norm_weight, void *y,
                                  float *states, void *stream);

/*
 * kda_chunk_prefill_states -- kda_chunk_prefill that also stores the state after every
 * token (the 'states' output of the nnterp Kimi-Linear page's support() table,
 * [batch, seq, heads, key_dim, value_dim]), computed through the chunked form rather than
 * token by token.  Within a chunk the recurrence unrolls to
 *     S_t = diag(exp(g_t)) S_{t-1} + k_t u_t^T
 * with u_t the rows of the chunk's corrected values U, which the state scan forms anyway
 * (nnterp Kimi-Linear page, Notes, "Loading": the prompt kernel carries the state from
 * chunk to chunk).  The scan stores U of every chunk in the workspace and the state after
 * each chunk's last position into `states`; one more launch writes every other position
 * from the state before its chunk (one work-group per chunk and head, independent of the
 * other chunks), so the call runs at the HBM write rate rather than at the token-by-token
 * kernel's per-token latency.
 *   states [B, T, H, dk, dv] fp32, 16-byte aligned: states[b, t, h] is S after token t
 *          (a padding token repeats the carried state; tokens of a packed batch at or past
 *          cu_seqlens[N] are not written).  64 KB per token and head.
 *   o      required (the gated norm, when asked for, runs over it as its own launch).
 *   workspace  at least kda_chunk_prefill_states_workspace_size(p, cu_seqlens != NULL)
 *          bytes: the prefill's workspace plus 16,384 bytes per chunk and head.
 * Other arguments, results and the precision are those of kda_chunk_prefill; the states
 * agree with the token-by-token recurrence to the chunked kernel's rounding (the state
 * after a chunk's last position is the same value final_state gets at a sequence end).
 * Only the bf16, dk = dv = 128 matrix-core kernel has this form: other shapes return
 * KDA_ERR_UNSUPPORTED (kda_recurrent_states covers them).  Errors as for kda_chunk_prefill,
 * KDA_ERR_NULL also for a NULL o or states.  Nothing is allocated.
 */
kda_status_t kda_chunk_prefill_states(const kda_params_t *p,
                                      const void *q, const void *k, const void *v,
                                      const float *g, const float *beta,
                                      const float *initial_state,
                                      const int32_t *cu_seqlens, const uint8_t *mask,
                                      void *o, float *final_state,
                                      const void *gate, const float *norm_weight, void *y,
                                      float *states, void *workspace, size_t workspace_bytes, void *stream);
/* Bytes of workspace kda_chunk_prefill_states needs; 0 for invalid params or a shape
 * without the chunked form.  (N + ceil(T / 32)) * H * 49168 + 256 with packing, otherwise
 * B * ceil(T / 32) * H * 49168 + 256. */
size_t kda_chunk_prefill_states_workspace_size(const kda_params_t *p, int32_t packed);

/*
 * kda_gated_rmsnorm -- y = w * x / sqrt(mean(x^2) + eps) * sigmoid(gate) over each row
 * of `width` features (one head).  x and gate: [rows, width] in in_dtype; weight:
 * [width] fp32 shared by every row; y: [rows, width] out_dtype.  width must be a power
 * of two in [8, 512].  y may alias x.
 */
kda_status_t kda_gated_rmsnorm(const void *x, const void *gate, const float *weight, void *y,
                               int64_t rows, int32_t width, float eps,
                               int32_t in_dtype, int32_t out_dtype, void *stream);

/* Problem description of the short convolution. */
typedef struct {
  int32_t B;             /* batch rows; 1 when cu_seqlens packs the sequences              */
  int32_t T;             /* tokens per row (packed total with cu_seqlens)                  */
  int32_t D;             /* channels per token (a multiple of 8), e.g. heads * head_dim    */
  int32_t num_seqs;      /* sequences: len(cu_seqlens)-1 with cu_seqlens, else ignored (=B) */
  int32_t width;         /* filter width W, 2..4 (4 in the pages' configuration)           */
  int32_t activation;    /* 1: SiLU after the filter (the pages' setting), 0: none         */
  int32_t in_dtype;      /* kda_dtype_t of x and of the carried state                      */
  int32_t out_dtype;     /* kda_dtype_t of y                                               */
} kda_conv_params_t;

/*
 * kda_short_conv -- the causal short convolution that runs over the projected queries,
 * keys and values in front of the KDA kernel (Kimi-K3 atlas, KDA layer page, kda-init
 * code: a ShortConvolution with activation 'silu' on each projection; nnterp Kimi-Linear
 * page, module tree: a Conv1d with one width-4 filter per channel, padding 3, no bias).
 * Per channel c and token t of a sequence:
 *     z = sum_{j<W} weight[c][j] * x[t-(W-1)+j][c],    y[t][c] = z * sigmoid(z)  (or z)
 * Inputs before a sequence's first token come from its carried state, oldest first.
 *
 *   x              [B, T, D]         in_dtype
 *   weight         [D, W]            fp32, 4-byte aligned; weight[c][W-1] meets the newest input
 *   initial_state  [N, W-1, D]       in_dtype, the W-1 inputs before each sequence (oldest
 *                                    first), or NULL for zeros (start of a prompt)
 *   cu_seqlens     [N + 1]           int32 device offsets of packed sequences (B == 1,
 *                                    p->num_seqs = N), or NULL; not together with mask
 *   mask           [B, T]            uint8, 0 = padding: output 0 and the token never enters
 *                                    the window (it is skipped), or NULL
 *   y              [B, T, D]         out_dtype; must not overlap x
 *   final_state    [N, W-1, D]       in_dtype: the last W-1 inputs of each sequence (with
 *                                    the carried state in front when a sequence is shorter),
 *                                    or NULL to skip.  It may be the same buffer as
 *                                    initial_state (decode: state updated in place).
 * N = B without cu_seqlens.  Tokens of a packed batch outside [0, cu_seqlens[N]) are not
 * written.  A decode step is a call with T = 1 and the state passed as both
 * initial_state and final_state.  x, y and the states must be 16-byte aligned.
 * Errors: KDA_ERR_NULL (params, x, weight or y NULL), KDA_ERR_SHAPE (sizes, activation),
 * KDA_ERR_DTYPE, KDA_ERR_ALIGN, KDA_ERR_CONFLICT (cu_seqlens with mask, cu_seqlens with
 * B != 1, y overlapping x), KDA_ERR_UNSUPPORTED (D not a multiple of 8, W outside 2..4,
 * more than 65535 rows, sequences or 64-token tiles), KDA_ERR_HIP.  Nothing is allocated.
 */
kda_status_t kda_short_conv(const kda_conv_params_t *p, const void *x, const float *weight,
                            const void *initial_state, const int32_t *cu_seqlens,
                            const uint8_t *mask, void *y, void *final_state, void *stream);

/*
 * The short convolution fused into the KDA kernels' prologue: the layer's q, k and v
 * projections each pass a causal width-W filter (then SiLU) right before the recurrence,
 * and the layer carries the last W-1 inputs of every sequence between calls, besides the
 * state (Kimi-K3 atlas, KDA layer page, kda-init code: ShortConvolution with activation
 * 'silu' on q, k and v; nnterp Kimi-Linear page, Notes on KDA: the convolution runs over
 * the projected queries, keys and values, so the mixer keeps its last tokens outside the
 * state).  The filter, the window rule (padding skipped, a sequence starting from its
 * carried inputs) and the carried inputs after the call are those of kda_short_conv, with
 * x = the raw q, k or v and D = H * d channels each (head h owns channels h*d .. h*d+d-1).
 * The filtered values stay in fp32 inside the kernels (a separate kda_short_conv pass would
 * store them in its out_dtype first): the fused call equals kda_short_conv with fp32 outputs
 * followed by the recurrence on those values, up to the recurrence kernels' own rounding.
 */
typedef struct {
  int32_t width;            /* W, 2..4 (4 in the pages' configuration)                        */
  int32_t activation;       /* 1: SiLU after the filter (the pages' setting), 0: none          */
  const float *weight_q;    /* [H * dk, W] fp32 taps per channel; weight[c][W-1] meets the     */
  const float *weight_k;    /*   newest input (as kda_short_conv's weight)                     */
  const float *weight_v;    /* [H * dv, W]                                                     */
  const void *initial_q;    /* [N, W-1, H * dk] in_dtype: the W-1 inputs before each sequence  */
  const void *initial_k;    /*   (oldest first), or NULL for zeros (start of a prompt)         */
  const void *initial_v;    /* [N, W-1, H * dv]                                                */
  void *final_q;            /* [N, W-1, H * d] in_dtype: the last W-1 inputs of each sequence  */
  void *final_k;            /*   after the call (padding skipped), or NULL to skip; each may   */
  void *final_v;            /*   be the same buffer as its initial_* (updated in place)        */
} kda_conv_t;

/*
 * kda_chunk_prefill_conv -- kda_chunk_prefill on the raw projections: q, k and v are the
 * inputs of the short convolution `conv`, which the kernels apply themselves (the
 * preparation filters q and k of each chunk, the scan filters v; the filtered values never
 * go to memory).  Every other argument, layout and rule as kda_chunk_prefill (same
 * workspace size); N = num_seqs with cu_seqlens, else B.  After the recurrence, one more
 * launch writes the carried inputs of every sequence whose final_* is set.
 * Kernel: the bf16 matrix-core prefill only (in_dtype bf16, dk = dv = 128, chunk 0, 32 or
 * 64, T * H * 128 < 2^31); other shapes return KDA_ERR_UNSUPPORTED (run kda_short_conv,
 * then kda_chunk_prefill).  All conv pointers are 16-byte aligned device memory owned by
 * the caller; nothing is allocated.  Errors: those of kda_chunk_prefill, KDA_ERR_NULL
 * (conv or a weight NULL), KDA_ERR_SHAPE (activation), KDA_ERR_UNSUPPORTED (width outside
 * 2..4, more than 65535 sequences, other kernels), KDA_ERR_ALIGN.
 */
kda_status_t kda_chunk_prefill_conv(const kda_params_t *p, const kda_conv_t *conv,
                                    const void *q, const void *k, const void *v,
                                    const float *g, const float *beta,
                                    const float *initial_state,
                                    const int32_t *cu_seqlens, const uint8_t *mask,
                                    void *o, float *final_state,
                                    const void *gate, const float *norm_weight, void *y,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_recurrent_step_conv -- kda_recurrent_step on the raw projections of the new tokens:
 * each token's q, k and v are filtered with the row's carried inputs (conv->initial_*,
 * [B, W-1, H * d]) in the kernel, and the carried inputs after the call go to
 * conv->final_* (decode: pass the same buffer as initial_* and final_*; the kernel that
 * owns a head updates its channels in place, or, when a head is split over several
 * work-groups, a second launch does).  A padding token (mask 0) leaves the window as it
 * is.  T = 0 only copies the carried inputs.  Other arguments, layout and errors as
 * kda_recurrent_step, plus those of kda_chunk_prefill_conv's conv checks.  Any dk = dv
 * that kda_recurrent_step takes.
 */
kda_status_t kda_recurrent_step_conv(const kda_params_t *p, const kda_conv_t *conv,
                                     const void *q, const void *k, const void *v,
                                     const float *g, const float *beta,
                                     float *state, const uint8_t *mask,
                                     void *o,
                                     const void *gate, const float *norm_weight, void *y,
                                     void *stream);

/*
 * kda_gated_norm_proj -- the layer's exit at decode: the sigmoid-gated RMSNorm of each
 * head's output, then the output projection (Kimi-K3 atlas, gate-project page: the heads
 * [B, 1, 96 x 128] leave as [B, 1, 7168]; Parameters table: gated RMSNorm 128, output
 * projection 88,080,384 = 12,288 x 7,168, no bias).
 *   o, gate      [rows, heads * head_dim]  bf16 (rows = B * T, heads side by side)
 *   norm_weight  [head_dim]                fp32, shared by all heads
 *   proj_weight  [out_features, heads * head_dim]  bf16 (the Linear layout [out, in])
 *   y            [rows, heads * head_dim]  bf16 output: the gated-normed heads (the
 *                                          projection's input; may alias o)
 *   out          [rows, out_features]      out_dtype: out = y proj_weight^T, fp32 accumulation
 *   workspace    device scratch of at least kda_out_proj_workspace_size(rows, heads *
 *                head_dim, out_features) bytes (fp32 partial sums when K is split), 16-byte
 *                aligned; may be NULL when that size is 0
 * head_dim a power of two in [8, 512]; heads * head_dim a multiple of 256; out_features a
 * multiple of 64; rows <= 65535 * 64.  The norm runs once per row and head, then the
 * projection (a fused per-tile norm would repeat the norm in every output tile); for
 * rows <= 64 the projection splits K and adds the partial sums in a fixed order.
 * All pointers 16-byte aligned device memory owned by the caller; nothing is allocated.
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_ALIGN, KDA_ERR_UNSUPPORTED,
 * KDA_ERR_WORKSPACE, KDA_ERR_HIP.
 */
kda_status_t kda_gated_norm_proj(const void *o, const void *gate, const float *norm_weight,
                                 const void *proj_weight, void *y, void *out, int64_t rows,
                                 int32_t heads, int32_t head_dim, int32_t out_features, float eps,
                                 int32_t out_dtype, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * kda_gated_norm_proj_noalloc -- kda_gated_norm_proj without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The split-K partial sums go to a
 * static device array of the library (16 MiB per GPU, held until the process ends), so
 * the call allocates nothing and needs no workspace; the caller still provides every
 * input and output.  Arguments, layout and the other errors as kda_gated_norm_proj.
 * Limit: the partials take 4 * S * rows * out_features bytes (S = 4 K slices for
 * rows <= 64 and heads * head_dim a multiple of 1024, S = 2 for a multiple of 512, no
 * partials otherwise); a call that needs more than 16 MiB returns KDA_ERR_WORKSPACE
 * (the decode exit, 64 rows x 7,168 features, needs 7.3 MB).  Every call on one GPU
 * shares that GPU's array, which keeps the last call's partials: calls that overlap in
 * time on one GPU (other streams, other threads) race and must not be issued.
 */
kda_status_t kda_gated_norm_proj_noalloc(const void *o, const void *gate, const float *norm_weight,
                                         const void *proj_weight, void *y, void *out, int64_t rows,
                                         int32_t heads, int32_t head_dim, int32_t out_features, float eps,
                                         int32_t out_dtype, void *stream);

/*
 * kda_out_proj -- the output projection alone: out[rows, out_features] = x W^T with
 * x [rows, in_features] bf16 and W [out_features, in_features] bf16 (Linear layout, no
 * bias), fp32 accumulation, out in out_dtype.  in_features a multiple of 256,
 * out_features a multiple of 64.  Pointers 16-byte aligned; workspace and errors as above.
 */
kda_status_t kda_out_proj(const void *x, const void *weight, void *out, int64_t rows,
                          int32_t in_features, int32_t out_features, int32_t out_dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace kda_out_proj and kda_gated_norm_proj need (0 when K is not split or
 * the sizes are unsupported). */
size_t kda_out_proj_workspace_size(int64_t rows, int32_t in_features, int32_t out_features);

/* Text of a status code (static storage). */
const char *kda_status_string(kda_status_t s);
/* Detail of the last non-OK status returned on this thread (thread-local storage). */
const char *kda_last_error(void);
/* Library version string, e.g. "kda-mi355x 0.1.0 gfx950". */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
