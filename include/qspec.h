/*
 * qspec.h -- C-ABI of libqspec.so, the MI355X (gfx950) hot path of QSpec-style
 * quantized speculative decoding with one shared INT4 weight set.
 *
 * Sources of the operations (pages):
 *   [P1] qiita.com, "QSpec実行時の2つの量子化による推論の一致率を調べる":
 *        sections "W4A16", "W4A4" and "QSpec の W4A4 モードと W4A16 モード" --
 *        one 4-bit weight set, run with 16-bit activations (verify) or with
 *        activations quantized to 4 bits at compute time (draft).
 *   [P3] kasblo.com, "Speculative Decodingとは？LLM生成を速くする方法":
 *        "draft modelとtarget modelの処理フロー" (draft gamma tokens, score gamma+1
 *        positions, accept left to right, stop at the first mismatch),
 *        "greedy decodingでは一致するprefixを採用する" (Top-1 prefix match),
 *        "samplingでもtargetの確率分布を保つ" (a(x) = min(1, p/q) and the residual
 *        max(0, p - q) normalised), "3 tokenの数値例" (worked example).
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or keeps a pointer after returning.
 *   - Tensors are dense row-major.  fp16 values travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on `stream` and returns; nothing synchronises.
 *     Buffers must stay alive until that work has completed.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     returned as a negative status; a launch failure returns QS_ERR_HIP.  A
 *     device-side fault surfaces at the caller's next synchronisation.  Nothing
 *     is printed and no exception crosses the ABI.
 *   - No global state besides cached device properties; calls on different
 *     streams may run concurrently if their output buffers do not overlap.
 *   - Shapes: K is a multiple of 128 (the weight group) and at most 65536;
 *     1 <= M <= 256 rows; N >= 1.  Weight buffers are padded to whole 16-row
 *     blocks (qs_packed_weight_bytes / qs_packed_scale_bytes).
 *   - Pointers to 16-byte vector data (x, w_packed, logits when V % 4 == 0)
 *     must be 16-byte aligned, else QS_ERR_MISALIGNED.
 */
#ifndef QSPEC_H
#define QSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QS_OK 0
#define QS_ERR_INVALID_ARG (-1) /* null pointer, bad shape, bad mode              */
#define QS_ERR_UNSUPPORTED (-2) /* shape outside the supported range (M > 256)    */
#define QS_ERR_MISALIGNED (-3)  /* vector-accessed pointer not 16-byte aligned    */
#define QS_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required     */
#define QS_ERR_HIP (-5)         /* the HIP runtime reported an error at launch    */
#define QS_ERR_DEVICE (-6)      /* current device is not a gfx950 (CDNA4) GPU     */

#define QS_GROUP 128   /* k-elements per weight scale group */
#define QS_MAX_M 256   /* most activation rows per linear call */
#define QS_MAX_VERIFY_SEQS 16384 /* sequences per verify launch block */

typedef enum { QS_W4A16 = 0, QS_W4A4 = 1, QS_W4A8 = 2 } qs_mode;

/* Human-readable text of a status code (static storage, never NULL). */
const char* qs_status_string(int status);

/* Bytes of the packed nibble buffer / packed scale buffer for an [N, K] weight. */
size_t qs_packed_weight_bytes(int N, int K);
size_t qs_packed_scale_bytes(int N, int K);

/*
 * qs_pack_weights -- re-lay one logical INT4 weight set into the layout both
 * linear modes stream ([P1] mode tree: a single 4-bit weight set serves the
 * W4A4 draft and the W4A16 verify).  Offline step, not on the timed path.
 *   q        int8 [N][K], codes in [-8, 7] (values outside are clamped)
 *   s        fp16 [N][K/128], scale of group g = k/128 of row n (symmetric,
 *            W[n][k] = q[n][k] * s[n][k/128])
 *   w_packed out, qs_packed_weight_bytes(N, K) bytes, 16-byte aligned
 *   s_packed out, qs_packed_scale_bytes(N, K) bytes
 * The packed layout is internal to the library; only the linear calls read it.
 */
int qs_pack_weights(const int8_t* q, const uint16_t* s, int N, int K,
                    uint8_t* w_packed, uint16_t* s_packed, void* stream);

/*
 * qs_linear_w4a16 -- verify-mode linear ([P1] "W4A16"): 4-bit weights are
 * expanded inside the kernel and multiplied with fp16 activations on fp16
 * MFMA with fp32 accumulation; each 128-wide group's partial sum is scaled in
 * fp32 (every row count: the products are exact, only the fp32 summation
 * order differs from the definition).
 *   x  fp16 [M][K];  y  fp32 [M][N] (out):  y[m][n] = sum_k x[m][k] * W[n][k]
 */
int qs_linear_w4a16(const uint16_t* x, const uint8_t* w_packed,
                    const uint16_t* s_packed, float* y, int M, int N, int K,
                    void* stream);

/*
 * Workspace bytes needed by qs_linear_w4a4 / qs_lmhead for these shapes: the
 * quantized activations and, for the batched kernel (W4A16 from 5 rows, W4A4
 * from 2), its K-split counters and partials.  0 when nothing is staged (one
 * W4A4 row, or W4A16 up to 4 rows).  A workspace given for a batched call is
 * cleared of stale counters by the call itself.
 */
size_t qs_linear_workspace_bytes(int mode, int M, int N, int K);

/*
 * qs_linear_w4a4 -- draft-mode linear ([P1] "W4A4"): activations are
 * quantized per token to INT4,
 *     s_m = fp16(fp32(max_k |x[m][k]|) / 7),  xq = clamp(rint(x / s_m), -8, 7)
 * (round half to even of the exact quotient; an all-zero row gives s_m = 0 and
 * xq = 0), then multiplied with the weight codes on int8 MFMA with i32
 * accumulation per 128-wide group:
 *     acc[m][n][g] = sum_{k in g} xq[m][k] * q[n][k]
 *     y[m][n]      = s_m * sum_g s[n][g] * acc[m][n][g]
 * The group sums are exact i32; y is formed in fp64, where every term and sum
 * is exact while log2(K/128) + (binades spanned by row n's scales) <= 17 (13
 * for W4A8), and rounded once to fp32: y is the exact value correctly rounded.
 *   x        fp16 [M][K];  y fp32 [M][N] (out)
 *   xq_out   optional int8 [M][K]   (NULL: not written)
 *   sx_out   optional fp16 [M]      (NULL: not written)
 *   acc_out  optional int32 [M][N][K/128] (NULL: not written)
 *   ws       workspace of at least qs_linear_workspace_bytes(QS_W4A4, M, N, K)
 *            bytes (may be NULL when that is 0); contents are scratch.
 */
int qs_linear_w4a4(const uint16_t* x, const uint8_t* w_packed,
                   const uint16_t* s_packed, float* y, int M, int N, int K,
                   int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * qs_linear_w4a8 -- the shared INT4 weights with 8-bit activations ([P2]
 * "3.中核となる技術的要素" names W4A8 beside W4A16 as a studied bit-width
 * configuration; the quantizer is this library's reading, the 4-bit one with
 * the int8 range):
 *     s_m = fp16(fp32(max_k |x[m][k]|) / 127),  xq = clamp(rint(x / s_m), -128, 127)
 * then the same int8-MFMA group sums and fp32 epilogue as qs_linear_w4a4
 * (|acc| <= 128 * 128 * 8).  Arguments, layouts, ownership and errors as for
 * qs_linear_w4a4; ws of qs_linear_workspace_bytes(QS_W4A8, M, N, K) bytes
 * (never 0: the codes are always staged).
 */
int qs_linear_w4a8(const uint16_t* x, const uint8_t* w_packed,
                   const uint16_t* s_packed, float* y, int M, int N, int K,
                   int8_t* xq_out, uint16_t* sx_out, int32_t* acc_out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * qs_lmhead -- the LM-head projection hidden -> vocabulary logits in any
 * mode (the pages' per-position next-token distributions, [P1] "結果", come from
 * it).  Same arithmetic as the linear of that mode with N = V.
 *   mode     QS_W4A16, QS_W4A4 or QS_W4A8
 *   x        fp16 [M][K];  logits fp32 [M][V] (out)
 *   ws       qs_linear_workspace_bytes(mode, M, V, K) bytes (NULL if 0)
 */
int qs_lmhead(int mode, const uint16_t* x, const uint8_t* w_packed,
              const uint16_t* s_packed, float* logits, int M, int V, int K,
              void* ws, size_t ws_bytes, void* stream);

/*
 * qs_lmhead_top1 -- the LM-head with a fused Top-1 epilogue: the logits of
 * qs_lmhead (written only if `logits` is not NULL) and, per row, the target's
 * Top-1 ([P1] "結果": each mode's Top-1 token and its probability; [P3]
 * greedy section) without a second pass over the logits:
 *   top1[m]      = argmax_v logits[m][v]   (lowest index among equal maxima)
 *   top1_prob[m] = 1 / sum_v exp(logits[m][v] - max)   (softmax, temperature 1)
 * Each wave of an output tile reduces its 64 columns of every row to (max,
 * sum of exp, first argmax); a second, small launch merges a row's partials
 * in column order.
 *   mode       QS_W4A16, QS_W4A4 or QS_W4A8 (arithmetic of that mode's linear)
 *   x          fp16 [M][K];  logits fp32 [M][V] (out, nullable)
 *   top1       int32 [M] (out);  top1_prob fp32 [M] (out, nullable)
 *   ws         >= qs_lmhead_top1_workspace_bytes(mode, M, V, K) bytes,
 *              zero-filled before its first use (its first bytes are arrival
 *              counters that every call leaves at zero); calls that overlap in
 *              time must not share it
 * Errors as qs_linear_w4a4; a missing or short workspace -> QS_ERR_WORKSPACE.
 */
size_t qs_lmhead_top1_workspace_bytes(int mode, int M, int V, int K);
int qs_lmhead_top1(int mode, const uint16_t* x, const uint8_t* w_packed,
                   const uint16_t* s_packed, float* logits, int M, int V, int K,
                   int32_t* top1, float* top1_prob,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * One linear of a chain (see qs_chain_forward).  Weights come from
 * qs_pack_weights; the struct itself is read on the host during the call.
 */
typedef struct qs_linear_desc {
  const uint8_t* w_packed;   /* packed codes of an [N, K] weight set          */
  const uint16_t* s_packed;  /* packed group scales                            */
  int N;                     /* output features                                */
  int K;                     /* input features (multiple of 128)               */
} qs_linear_desc;

/* Workspace bytes needed by qs_chain_forward for this chain at M rows. */
size_t qs_chain_workspace_bytes(int mode, int M, const qs_linear_desc* chain, int n);

/*
 * qs_chain_forward -- one forward pass of a stack of quantized linears in one
 * mode: the W4A4 draft pass at M = batch rows or the W4A16 verify pass at
 * M = batch * (gamma + 1) rows, where the target scores all candidate positions
 * in a single pass ([P3] "draft modelとtarget modelの処理フロー"; [P1] mode tree).
 * The pages give no layer internals, so the chain is linears only:
 *   stage 0 reads x fp16 [M][chain[0].K];
 *   stage i > 0 reads v = the first chain[i].K columns (row stride
 *     chain[i-1].N) of stage i-1's output, kept as fp16 in the workspace, and
 *     standardises each row of v over those columns, (v - mean) / std with the
 *     population std (rows with zero spread become zeros), standing in for the
 *     normalisation between real layers (requires chain[i].K <= chain[i-1].N);
 *   the last stage writes fp32 out [M][chain[n-1].N].
 * Arithmetic, the same for every row count and launch configuration:
 *   W4A16: the fp16 rows v are the 16-bit activations of the product; the
 *     standardisation is folded into the epilogue, y = (sum_k v w - mean *
 *     sum_k w) / std, with fp32 row statistics; a stage output is fp16(y).
 *   W4A4, W4A8: the standardised row is rounded to fp16 (statistics and value
 *     in fp64, one correct rounding) and quantized as in the single linear;
 *     y is exact (see qs_linear_w4a4) and rounded once to the fp16 stage
 *     output or the fp32 result -- every code, group sum and stage value is
 *     the float64 definition's own.
 * With chain = n_layers x {q|k|v, o, gate|up, down} + LM-head this is the
 * Llama-shaped pass: o reads the q columns, down reads the gate columns.
 *   ws  >= qs_chain_workspace_bytes(mode, M, chain, n) bytes of scratch
 */
int qs_chain_forward(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n,
                     float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * qs_chain_forward_top1 -- qs_chain_forward whose last stage (the LM-head) also
 * reduces each row of its output to the target's Top-1 inside its epilogue
 * ([P1] "結果": each mode's Top-1 token and its probability; [P3] greedy
 * section: greedy acceptance needs only the target's argmax per position), so
 * a greedy verify needs no second pass over the logits:
 *   top1[m]      = argmax_v y[m][v]   (lowest index among equal maxima)
 *   top1_prob[m] = 1 / sum_v exp(y[m][v] - max)   (softmax, temperature 1)
 * over the fp32 values y that out receives (the same values as
 * qs_chain_forward's out, whose arithmetic this call shares).
 *   out        fp32 [M][chain[n-1].N] (out, nullable: the logits are then not
 *              written)
 *   top1       int32 [M] (out);  top1_prob fp32 [M] (out, nullable)
 *   ws         >= qs_chain_top1_workspace_bytes(mode, M, chain, n) bytes of
 *              scratch (no zero-fill needed)
 * The persistent pass reduces each workgroup's columns to one partial per row
 * and the last workgroup to finish merges them; on the per-linear path the
 * LM-head runs as in qs_lmhead_top1 (partials per wave, then a merge launch).  After a persistent-pass wait
 * time-out (see qs_set_barrier_timeout_us) top1 holds -1 and top1_prob NaN
 * for every row whose merge did not run.  Errors as qs_chain_forward.
 */
size_t qs_chain_top1_workspace_bytes(int mode, int M, const qs_linear_desc* chain, int n);
int qs_chain_forward_top1(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n,
                          float* out, int32_t* top1, float* top1_prob,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Number of persistent pass-kernel launches qs_chain_forward makes for this
 * chain on the current device (each runs a run of consecutive linears with
 * grid-wide hand-over between them), or 0 if the chain runs one linear per
 * launch (row counts or shapes the persistent kernel does not take).  The
 * persistent launches of a pass are preceded by one launch that clears the
 * control words and (W4A4, W4A8) fills the stage outputs with the
 * not-yet-written pattern (and, W4A4 above one row, the shared activation
 * codes).  Negative status codes as qs_chain_forward for bad arguments.
 */
int qs_chain_pass_launches(int mode, int M, const qs_linear_desc* chain, int n);

/*
 * Wall-clock limit, in microseconds, of every wait inside a persistent pass
 * (W4A16: a grid-barrier wait; W4A4 and W4A8: the wait for one stage's input,
 * or for its shared activation codes, to be written) (process-wide; default
 * 200000).  A wait that passes it sets
 * the workspace's time-out word and the workgroup exits, so a pass can never
 * wait forever.  The output is then partly or wholly NaN: every value is
 * either the correct one or NaN (the pass fills its output with NaN before it
 * starts, and a workgroup writes only after all its waits succeeded), so no
 * value from an earlier call survives.  0 makes every wait fail at once, which
 * exercises that path.  QS_ERR_INVALID_ARG if us < 0.
 */
int qs_set_barrier_timeout_us(int us);

/*
 * Whether the last qs_chain_forward call on this workspace (same chain and
 * arguments) had a wait time out: *timed_out = 1 if so, else 0.
 * Synchronises `stream`.  The word is cleared by the next persistent
 * qs_chain_forward on the workspace.  Chains that run one launch per linear
 * always report 0.  Errors as qs_chain_forward.
 */
int qs_chain_pass_status(int mode, int M, const qs_linear_desc* chain, int n, void* ws,
                         size_t ws_bytes, int* timed_out, void* stream);

/*
 * Measurement helpers of the persistent pass, for profiling the stage
 * hand-over; they compute nothing the pages define beyond qs_chain_forward.
 *
 * qs_chain_trace_bytes -- bytes of the timestamp buffer of qs_chain_forward_trace
 * for this chain and row count: entries x workgroups x 4 x 8, where entries is
 * the number of stage-table entries of the pass (a linear, or one K chunk of a
 * linear) and workgroups the number of compute units.  0 when the row count
 * does not run as a persistent pass (or for invalid arguments).
 *
 * qs_chain_forward_trace -- qs_chain_forward (same arguments, workspace, output
 * and errors), and in addition writes to the device buffer trace
 * (uint64 [entries][workgroups][4], trace_bytes >= qs_chain_trace_bytes,
 * 16-byte aligned, owned by the caller) the device wall-clock (the 100 MHz
 * realtime counter, read by each workgroup's first control thread) at four
 * points of every entry:
 *   [0] the entry's input is staged in LDS (its streaming may start);
 *   [1] the streaming waves have parked the entry's partial sums;
 *   [2] the entry's outputs are stored (W4A16: all of the workgroup's stores
 *       acknowledged; the integer modes: the first control wave's stores issued);
 *   [3] the hand-over is done (W4A16: all workgroups' arrival flags seen; equal
 *       to [2] where no grid barrier follows).
 * The timestamps cost one store each; results equal qs_chain_forward's.
 * QS_ERR_UNSUPPORTED when the row count runs one launch per linear.
 */
size_t qs_chain_trace_bytes(int mode, int M, const qs_linear_desc* chain, int n);
int qs_chain_forward_trace(int mode, const uint16_t* x, int M, const qs_linear_desc* chain, int n,
                           float* out, void* ws, size_t ws_bytes, unsigned long long* trace,
                           size_t trace_bytes, void* stream);

/*
 * Workspace bytes for qs_verify_greedy / qs_verify_sample at (B, gamma, V);
 * 0 for arguments out of range (gamma > 63).  A batch of more than
 * QS_MAX_VERIFY_SEQS sequences runs as consecutive blocks of at most that many
 * on the stream, so the size stops growing there.
 *
 * A verify workspace must be zero-filled once before its first use: its first
 * 4 MiB hold per-sequence arrival counters (the last workgroup of a sequence
 * to arrive finishes it within the same launch), and every call leaves them at
 * zero again, so one workspace can then serve any sequence of calls and shapes
 * on one stream.  Calls that overlap in time must not share a workspace.
 */
size_t qs_verify_workspace_bytes(int B, int gamma, int V);

/*
 * qs_verify_greedy -- Top-1 and greedy prefix-match acceptance ([P3] greedy
 * section; [P1] "Speculative Decoding": a mismatching draft token is replaced by
 * the target's own Top-1).  Per sequence b:
 *   t[i]      = argmax_j tgt_logits[b][i][j] (lowest index among equal maxima)
 *   top1_prob = 1 / sum_j exp(l_j - l_max)   (softmax at temperature 1)
 *   n         = number of leading i < gamma with draft_ids[b][i] == t[i]
 *   out_tokens[b] = draft_ids[b][0..n-1], t[n], then -1 up to gamma+1 entries
 * gamma = 0 is a plain Top-1 (the draft step): out_tokens[b][0] = t[0].
 *   tgt_logits fp32 [B][gamma+1][V];  draft_ids int32 [B][gamma] (ids outside
 *   [0, V) are mismatches and are never used as addresses; may be NULL if gamma = 0)
 *   tgt_top1   int32 [B][gamma+1] (out);  top1_prob fp32 [B][gamma+1] (out, nullable)
 *   n_accept   int32 [B] (out);  out_tokens int32 [B][gamma+1] (out)
 *   ws         >= qs_verify_workspace_bytes(B, gamma, V) bytes of scratch,
 *              zero-filled before its first use (see qs_verify_workspace_bytes)
 */
int qs_verify_greedy(const float* tgt_logits, const int32_t* draft_ids,
                     int B, int gamma, int V,
                     int32_t* tgt_top1, float* top1_prob,
                     int32_t* n_accept, int32_t* out_tokens,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * qs_accept_greedy -- the prefix rule of qs_verify_greedy ([P3] "greedy
 * decodingでは一致するprefixを採用する"; [P1] "Speculative Decoding") applied to
 * Top-1 ids already computed, e.g. by qs_chain_forward_top1 over the verify
 * pass's B * (gamma + 1) rows:
 *   n = number of leading i < gamma with draft_ids[b][i] == tgt_top1[b][i]
 *   out_tokens[b] = draft_ids[b][0..n-1], tgt_top1[b][n], then -1 up to
 *   gamma + 1 entries;  n_accept[b] = n
 *   tgt_top1   int32 [B][gamma+1];  draft_ids int32 [B][gamma] (may be NULL
 *              if gamma = 0);  n_accept int32 [B] (out);  out_tokens int32
 *              [B][gamma+1] (out)
 * A negative tgt_top1 entry (what a timed-out pass leaves) matches nothing.
 * One thread per sequence, no workspace.  gamma > 63 -> QS_ERR_UNSUPPORTED.
 */
int qs_accept_greedy(const int32_t* tgt_top1, const int32_t* draft_ids, int B, int gamma,
                     int32_t* n_accept, int32_t* out_tokens, void* stream);

/*
 * qs_verify_greedy_noalloc -- qs_verify_greedy for callers that cannot
 * allocate or pass device memory of their own: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * outputs and errors, without the workspace: its scratch (arrival counters and
 * statistics partials) is a fixed device array inside the library, one per
 * GPU, of qs_verify_greedy_noalloc_max_bytes() bytes (8 MiB), held until the
 * process ends.  A call whose qs_verify_workspace_bytes(B, gamma, V) exceeds
 * that returns QS_ERR_UNSUPPORTED before any device work.  The call allocates
 * nothing; a device's first call also clears the counters (with a kernel on
 * `stream`), and every call leaves them cleared.  All calls on one GPU share
 * the array: calls that overlap in time on the same GPU race.
 */
size_t qs_verify_greedy_noalloc_max_bytes(void);
int qs_verify_greedy_noalloc(const float* tgt_logits, const int32_t* draft_ids,
                             int B, int gamma, int V,
                             int32_t* tgt_top1, float* top1_prob,
                             int32_t* n_accept, int32_t* out_tokens,
                             void* stream);

/*
 * qs_verify_tree_greedy -- greedy acceptance over a tree of draft candidates
 * scored in one target pass ([P2] "3.中核となる技術的要素": verification that
 * expands into a tree; the rule is this library's reading, the greedy prefix
 * rule of [P3] "greedy decodingでは一致するprefixを採用する" applied along every
 * root-to-node path).  Per sequence b, with T nodes, node 0 the root (the last
 * committed token):
 *   t[i]   = argmax_j tgt_logits[b][i][j] (lowest index among equal maxima),
 *            the target's choice after node i
 *   node i >= 1 is accepted iff 0 <= parent[b][i] < i, its parent is accepted
 *            and tokens[b][i] == t[parent[b][i]]; the root is accepted
 *   winner = the deepest accepted node (lowest index on equal depth); n = its depth
 *   out_tokens[b] = the tokens along the root-to-winner path, t[winner], then -1
 *   out_nodes[b]  = the path's nodes (root excluded), then -1
 * A chain (parent[i] = i - 1) is qs_verify_greedy with gamma = T - 1.
 *   tgt_logits fp32 [B][T][V];  tokens, parent int32 [B][T] (entry 0 unused;
 *              out-of-range tokens or parents never match and are never used as
 *              addresses; both may be NULL if T = 1)
 *   tgt_top1   int32 [B][T] (out);  n_accept int32 [B] (out)
 *   out_tokens int32 [B][T] (out);  out_nodes int32 [B][T] (out, nullable)
 *   ws         >= qs_verify_workspace_bytes(B, T - 1, V) bytes, zero-filled
 *              before its first use (see qs_verify_workspace_bytes)
 * Errors: T < 1 or a NULL required pointer -> QS_ERR_INVALID_ARG; T > 64 ->
 * QS_ERR_UNSUPPORTED; workspace too small -> QS_ERR_WORKSPACE.
 */
int qs_verify_tree_greedy(const float* tgt_logits, const int32_t* tokens,
                          const int32_t* parent, int B, int T, int V,
                          int32_t* tgt_top1, int32_t* n_accept,
                          int32_t* out_tokens, int32_t* out_nodes,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * qs_verify_sample -- sampling acceptance with residual resampling ([P3]
 * sampling section and its A/B/C example).  Per sequence b, with
 * p_i = softmax(tgt_logits[b][i]) (i <= gamma) and q_i = softmax(drf_logits[b][i]):
 *   a_i = min(1, p_i(d_i) / q_i(d_i)) for every i < gamma
 *         (p_i(d_i) = 0 -> 0; q_i(d_i) = 0 < p_i(d_i) -> 1; d_i outside [0,V) -> 0)
 *   n   = first i with u_accept[b][i] >= a_i (accept iff u < a), else gamma
 *   f   = max(0, p_n - q_n) / sum(max(0, p_n - q_n)) if n < gamma
 *         (falls back to p_n if that sum is 0), else p_gamma
 *   y   = smallest j with sum_{k<=j} f_k > u_final[b]  (inverse CDF; if rounding
 *         leaves none, the last j with f_j > 0)
 *   out_tokens[b] = d_0..d_{n-1}, y, then -1 padding;  n_accept[b] = n
 *   tgt_logits fp32 [B][gamma+1][V];  drf_logits fp32 [B][gamma][V]
 *   draft_ids int32 [B][gamma];  u_accept fp32 [B][gamma] in [0,1);  u_final fp32 [B]
 *   accept_prob fp32 [B][gamma] (out);  n_accept int32 [B] (out)
 *   out_tokens int32 [B][gamma+1] (out);  final_dist fp32 [B][V] (out, nullable) = f
 *   ws >= qs_verify_workspace_bytes(B, gamma, V) bytes of scratch, zero-filled
 *   before its first use (see qs_verify_workspace_bytes)
 * gamma = 0 draws one token from p_0 with u_final (drf_logits, draft_ids,
 * u_accept and accept_prob may then be NULL).
 */
int qs_verify_sample(const float* tgt_logits, const float* drf_logits,
                     const int32_t* draft_ids, const float* u_accept,
                     const float* u_final, int B, int gamma, int V,
                     float* accept_prob, int32_t* n_accept, int32_t* out_tokens,
                     float* final_dist, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSPEC_H */
