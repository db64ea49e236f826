/*
 * gdn.h -- C ABI of libgdn.so: the pooled Gated DeltaNet decode step for
 * MI355X (gfx950), its conv decode, and slot commit.
 *
 * Sources (the mstar pull-request pages):
 *   PR #1139, "Why" and "Numbers": the GDN rule of a Qwen3.5 decode step is
 *     state traffic -- the recurrent state is read from the pool and written
 *     back once per step, and writing a second slot instead of the one just
 *     read is cheaper.
 *   PR #1139, "What changed": a request holds two slots (twin_slots); a decode
 *     step reads one and writes the other, commit swaps them; prefill, split
 *     walks and the mixed step's decode half update in place (keep_in_place);
 *     both give the same values.  causal_conv1d_decode advances the conv
 *     window by one token a row and honours a separate write slot.
 *   PR #1139, "Tests", and PR #965, "What changed": padding rows address the
 *     null slot 0 and leave every real row's result unchanged.
 *   PR #965 review notes: a captured step must not allocate.
 *   The update rule is Gated DeltaNet's (Yang et al., ICLR 2025); the pages
 *   name it but never print it.
 *
 * Conventions for every entry point:
 *   - Every array pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees, synchronises the host or reads device
 *     memory from the host, so every call is stream-ordered on `stream` and
 *     can be captured into a HIP graph.
 *   - bf16 values travel as their 16-bit patterns (gdn_bf16).
 *   - Arguments are validated on the host before anything is launched; a
 *     non-OK status means nothing was enqueued (GDN_ERR_HIP: the launch
 *     itself failed).
 *   - Preconditions NOT checked on the host (they live in device memory):
 *     slot values lie in [0, N); no two real rows share a slot; for a twin
 *     write a real row's write slot differs from its read slot and from every
 *     other row's slots.  The kernels bounds-check every slot they read: a
 *     row with a slot outside [0, N), or a real row (read slot not 0) of a
 *     twin write whose write slot equals its read slot or is the null slot
 *     0, touches no pool memory and gets NaN in every output element
 *     instead.  Slot 0 is never written by any entry point.
 *     gdn_check_slots verifies the preconditions on the device, for
 *     debugging.
 *   - Calls that overlap on the same pool slots race (as any two kernels
 *     writing the same memory would).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t gdn_bf16; /* bfloat16 bit pattern */

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes or strides */
    GDN_ERR_UNSUPPORTED = 3, /* sizes outside what the kernels are built for */
    GDN_ERR_REFUSED = 4,     /* a twin-slot write with more than one token a row */
    GDN_ERR_HIP = 5,         /* the HIP launch returned an error */
    GDN_ERR_SCRATCH = 6      /* gdn_prefill_two_pass_noalloc: more scratch than its static buffer */
} gdn_status;

/* Sizes of one decode step.
 *   B    rows (requests) in the step; 0 is allowed, enqueues nothing and
 *        returns GDN_OK before any other check (the arrays may then be NULL)
 *   T    tokens per row, processed in order (T > 1 only in place)
 *   H_k  key heads;  H_v value heads, a multiple of H_k; value head hv reads
 *        key head hv / (H_v / H_k)
 *   d_k, d_v  head dims, each 64 or 128
 *   W    conv width (4)
 *   N    slots in the pool, including the null slot 0
 * The conv runs over C = 2*H_k*d_k + H_v*d_v channels ordered q | k | v,
 * head-major. */
typedef struct gdn_dims {
    int32_t B, T, H_k, H_v, d_k, d_v, W, N;
} gdn_dims;

/*
 * gdn_decode_step -- one fused GDN decode step over B rows of a slot pool
 * (PR #1139, "What changed": twin slots and keep_in_place; "Tests": padding
 * on the null slot; Gated DeltaNet's rule for the update).
 *
 * For each row r with rs = read_slot[r] and ws = write_slot[r] (ws = rs when
 * write_slot is NULL, the in-place mode), for t = 0..T-1, all in fp32:
 *   conv:   for each channel c, win = [conv_state[rs][0..W-2][c], x[r][t][c]],
 *           y[c] = silu(sum_w conv_w[c][w] * win[w] (+ conv_b[c])); the
 *           window advances by one token
 *   split:  q = y[hk*d_k ..], k = y[H_k*d_k + hk*d_k ..],
 *           v = y[2*H_k*d_k + hv*d_v ..], hk = hv / (H_v/H_k)
 *   norm:   q^ = q / sqrt(sum q^2 + l2_eps) * q_scale, k^ = k / sqrt(sum k^2 + l2_eps)
 *   rule:   alpha = exp(g[r][t][hv]), b = beta[r][t][hv]
 *           S <- alpha * S;  S <- S + b * k^ (v - S^T k^)^T;  o = S^T q^
 *   out[r][t][hv][:] = o rounded to bf16 (nearest even)
 * then S goes to state[ws] and the advanced window to conv_state[ws].
 * A row with rs == 0 is padding: its out is +0.0 and it reads and writes no
 * slot, so slot 0 stays as it is.
 *
 * Layouts (all contiguous unless a stride is given):
 *   x          [B][T][C] bf16; rows x_row_stride elements apart (>= T*C)
 *   conv_w     [C][W] bf16;  conv_b [C] bf16 or NULL
 *   conv_state [N][W-1][C] bf16 (oldest input first)
 *   state      [N][H_v][d_k][d_v] fp32, S[i][j] with i over keys
 *   g, beta    [B][T][H_v] fp32 (log decay, and the delta-rule strength)
 *   read_slot, write_slot  [B] int32; write_slot NULL => in place
 *   out        [B][T][H_v][d_v] bf16
 * Twin mode reads only read slots and writes only write slots and out; in
 * place reads and writes the read slots.  T > 1 with a twin write returns
 * GDN_ERR_REFUSED (multi-token walks stay in place).  In place needs
 * H_v/H_k in {1, 2, 4}.  Alignment (GDN_ERR_UNSUPPORTED otherwise): state
 * and conv_w 16 bytes; x, conv_b, conv_state and out 8 bytes; x_row_stride a
 * multiple of 4 elements.  Size limits (GDN_ERR_SHAPE otherwise): a row's x
 * with eight more tokens, its out and its gates each under 2 GiB, and conv_w
 * under 2 GiB.
 */
gdn_status gdn_decode_step(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                           const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state,
                           float *state, const float *g, const float *beta,
                           const int32_t *read_slot, const int32_t *write_slot, gdn_bf16 *out,
                           float q_scale, float l2_eps, hipStream_t stream);

/*
 * gdn_decode_step_commit -- gdn_decode_step (twin-slot write) with the
 * commit folded in (PR #1139, "What changed": commit swaps the two slots of
 * a request; "Numbers": a small kernel in a captured graph costs about as
 * much as its launch, so the step does it instead of a second kernel).
 * Everything gdn_decode_step does, plus, for every row r (padding rows
 * included):
 *   next_read_slot[r] = write_slot[r];  next_write_slot[r] = read_slot[r]
 * so the next step reads what this one wrote.  The next-step arrays must not
 * overlap read_slot or write_slot (the step reads those while it writes the
 * next ones); a caller alternates between two pairs of slot arrays.
 * write_slot, next_read_slot and next_write_slot are required (NULL gives
 * GDN_ERR_NULL); passing the same array twice gives GDN_ERR_SHAPE.
 */
gdn_status gdn_decode_step_commit(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                  const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state,
                                  float *state, const float *g, const float *beta, const int32_t *read_slot,
                                  const int32_t *write_slot, int32_t *next_read_slot, int32_t *next_write_slot,
                                  gdn_bf16 *out, float q_scale, float l2_eps, hipStream_t stream);

/*
 * gdn_decode_step_tokens -- T tokens a row from the read slot, keeping the
 * state after every token in a slot of its own, for speculative decoding's
 * verify pass (PR #1139, "What changed": speculative decoding's slots already
 * hold a state per token, which is why the pool refuses twin slots with it).
 *
 * For each row r with rs = read_slot[r]: the state S and conv window start
 * from slot rs; tokens t = 0..T-1 run in order exactly as in
 * gdn_decode_step; after token t, when ts = token_slots[r*T + t] is not 0,
 * the state and the advanced window at that point are stored to slot ts
 * (state[ts], conv_state[ts]).  out [B][T][H_v][d_v] gets every token's
 * read-out.  Slot rs itself is never written, so rejecting draft tokens costs
 * nothing: the caller keeps the slot of the last accepted token.
 * A row with rs == 0 is padding (out +0.0, no slot touched).  A row whose
 * read slot or any token slot lies outside [0, N), or has a token slot equal
 * to its read slot, touches no slot and gets NaN in out.
 * Layouts, sizes, alignment and errors as gdn_decode_step in place (write
 * slot NULL, H_v/H_k in {1, 2, 4}); token_slots is [B][T] int32 on the
 * device (NULL with B > 0: GDN_ERR_NULL).  Preconditions, not checked: the
 * non-zero token slots are distinct and are not any row's read slot.
 */
gdn_status gdn_decode_step_tokens(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                  const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state,
                                  float *state, const float *g, const float *beta, const int32_t *read_slot,
                                  const int32_t *token_slots, gdn_bf16 *out, float q_scale, float l2_eps,
                                  hipStream_t stream);

/*
 * gdn_prefill -- chunked prefill of packed prompts, each updating its slot in
 * place (PR #1139, "What changed": prefill keeps the state in place; PR #965
 * names the chunked GDN path that the mixed step's prompt rows take).
 *
 * dims: B = sequences, T = total tokens in x, g, beta and out (the packed
 * length); H_k, H_v, d_k, d_v, W, N as for gdn_decode_step.  Sequence b owns
 * tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of the packed arrays and slot
 * s = slot[b].  The result is what gdn_decode_step in place computes over
 * those tokens one after the other (conv decode + SiLU from the slot's
 * window, L2 norms, the gated delta rule from the slot's state, a read-out per
 * token), and the final state and window go back to slot s; the arithmetic is
 * the chunked form of that recurrence in fp32 (32-token chunks, matrix-core
 * products), so results match the token-by-token path within rounding, not
 * bit for bit.  s == 0 is a padding sequence: its read-out is +0.0 and no slot
 * is touched.  A sequence whose token range is not inside [0, T] or whose
 * slot is outside [0, N) touches nothing (its read-out is left as it was).
 *
 * Layouts: x [T][C] bf16, rows x_row_stride elements apart (>= C, even);
 * cu_seqlens [B+1] int32 and slot [B] int32 on the device; g, beta [T][H_v]
 * fp32; out [T][H_v][d_v] bf16; conv_w, conv_b, conv_state, state as for
 * gdn_decode_step.  Alignment (GDN_ERR_UNSUPPORTED otherwise): x and
 * conv_state 4 bytes, state 16.  Preconditions, not checked: no two
 * sequences share a slot; cu_seqlens is non-decreasing.
 */
gdn_status gdn_prefill(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride, const int32_t *cu_seqlens,
                       const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state, float *state,
                       const float *g, const float *beta, const int32_t *slot, gdn_bf16 *out, float q_scale,
                       float l2_eps, hipStream_t stream);

/*
 * gdn_prefill_two_pass -- the same computation and contract as gdn_prefill,
 * in two passes with a caller-provided workspace.  The first pass works on
 * every 32-token chunk of every prompt at once (conv decode + SiLU, L2 norms,
 * the chunk's decay and the triangular solve of the chunked delta rule,
 * PR #1139 "What changed": prefill in place), the second walks each prompt's
 * chunks in order.  Under 256 prompt-head pairs (B H_v) the first pass also
 * forms every product of a chunk that does not depend on the state and the
 * second splits each head's d_v columns over several workgroups (a single
 * long prompt fills the chip); from 256 pairs up (with the last round of 256
 * at least three quarters full) the first pass keeps only the chunk's solve
 * and per-token factors and the second, a workgroup per prompt and head, runs
 * the conv again from x (an eighth of the workspace).  When the second pass's
 * workgroups would fill at most half the compute units (one long prompt) and
 * the call has 64 chunks or more, the chunks go in consecutive ranges of 32
 * and the first pass of a range runs beside the walk of the one before: more
 * launches, the same bits (a prompt's state goes through its slot between
 * ranges unchanged).
 * Results match gdn_prefill within rounding, not bit for bit.
 *
 * workspace: device memory of at least
 * gdn_prefill_two_pass_workspace_bytes(dims) bytes, 256-byte aligned, owned
 * by the caller; its contents on entry do not matter and on return are
 * scratch.  Calls that share a workspace must be stream-ordered.  Beyond
 * gdn_prefill's statuses: GDN_ERR_NULL without a workspace,
 * GDN_ERR_UNSUPPORTED if it is misaligned, GDN_ERR_SHAPE if it is too small.
 */
gdn_status gdn_prefill_two_pass(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                const int32_t *cu_seqlens, const gdn_bf16 *conv_w, const gdn_bf16 *conv_b,
                                gdn_bf16 *conv_state, float *state, const float *g, const float *beta,
                                const int32_t *slot, gdn_bf16 *out, float q_scale, float l2_eps, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_prefill_two_pass_noalloc -- gdn_prefill_two_pass with no workspace
 * argument and no allocation at all, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same computation, kernels and results as
 * gdn_prefill_two_pass, bit for bit.
 *
 * Its scratch is a static device buffer of GDN_NOALLOC_SCRATCH_BYTES (64 MiB)
 * inside the library: every GPU the library is loaded on holds one copy until
 * the process ends, and the address of the current device's copy is looked up
 * on the first call on that device.  A call whose workspace
 * (gdn_prefill_two_pass_workspace_bytes of the same dims) exceeds it returns
 * GDN_ERR_SCRATCH and enqueues nothing: at 16 value heads of 128 x 128 that
 * is 1,888 tokens for one prompt, 32 fewer for each further prompt, while
 * a call of 16 such prompts (256 prompt-head pairs: the slim workspace)
 * holds 14,752 tokens.  Every
 * call on a GPU shares that GPU's buffer, so calls that overlap on one GPU
 * (on different streams, or from different threads without stream order
 * between them) race; calls ordered on one stream do not.  The buffer's
 * contents on entry do not matter.  Other statuses as gdn_prefill_two_pass
 * (GDN_ERR_HIP also if the buffer's address cannot be had).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_two_pass_noalloc(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                        const int32_t *cu_seqlens, const gdn_bf16 *conv_w, const gdn_bf16 *conv_b,
                                        gdn_bf16 *conv_state, float *state, const float *g, const float *beta,
                                        const int32_t *slot, gdn_bf16 *out, float q_scale, float l2_eps,
                                        hipStream_t stream);

/*
 * gdn_prefill_two_pass_workspace_bytes -- the workspace gdn_prefill_two_pass
 * needs for dims (B sequences, T packed tokens, H_k, H_v, d_k, d_v): room for
 * K = ceil(T / 32) + B chunks (every sequence adds at most one partial chunk)
 * per value head, each chunk (3 d_k + d_v + 32) * 32 + 1 fp32 values in the
 * full layout, 2 * 32 * 32 + 128 fp32 values in the slim one (B H_v at least
 * 256, the last round of 256 at least three quarters full), plus in that
 * case B * 3 * C bf16 (C = 2 H_k d_k + H_v d_v, a copy of each prompt's
 * window); plus B + 1 int32 and 4 int32 per chunk; each region rounded up to
 * 256 bytes.  0 when dims is NULL or its sizes are unusable.
 */
size_t gdn_prefill_two_pass_workspace_bytes(const gdn_dims *dims);

/*
 * conv_decode -- the pooled conv update for one token a row, standalone
 * (PR #1139, "What changed": causal_conv1d_decode, with null slots, strided
 * rows, optional bias and activation, and a write slot that leaves the read
 * slot alone).
 *
 * For each row r with rs = read_slot[r], ws = write_slot ? write_slot[r] : rs,
 * and each channel c < C:
 *   win = [conv_state[rs][0..W-2][c], x[r][c]]
 *   y   = sum_w conv_w[c][w] * win[w] (+ conv_b[c]), in fp32
 *   out[r][c] = bf16(activation ? silu(y) : y)
 *   conv_state[ws][..][c] = win[1..W-1]   (a bit-exact shift of bf16 values)
 * A row with rs == 0 gets +0.0 outputs and touches no slot.  A row with
 * rs != 0 and a slot outside [0, N), or with ws == 0 (the null slot never
 * holds a window), gets NaN outputs and touches no slot.
 *   x   [B][C] bf16, rows x_row_stride elements apart (>= C)
 *   out [B][C] bf16, rows out_row_stride elements apart (>= C)
 *   activation: 0 none, 1 SiLU.  W must be 4.  B = 0 returns GDN_OK at once.
 */
gdn_status conv_decode(int32_t B, int32_t C, int32_t W, int32_t N, const gdn_bf16 *x,
                       int64_t x_row_stride, const gdn_bf16 *conv_w, const gdn_bf16 *conv_b,
                       gdn_bf16 *conv_state, const int32_t *read_slot, const int32_t *write_slot,
                       gdn_bf16 *out, int64_t out_row_stride, int32_t activation,
                       hipStream_t stream);

/*
 * slot_commit -- commit of a twin-slot step (PR #1139, "What changed"): each
 * row's read and write slot trade places on the device, stream-ordered after
 * the step, so the next step reads what this one wrote.  Rows whose two
 * slots are equal (in place, padding on slot 0) are unchanged.
 *   read_slot, write_slot [B] int32.  B = 0 returns GDN_OK at once.
 */
gdn_status slot_commit(int32_t *read_slot, int32_t *write_slot, int32_t B, hipStream_t stream);

/*
 * gdn_check_slots -- a debug check, on the device, of the slot preconditions
 * every decode step relies on and does not verify (PR #1139, "What changed":
 * a step reads one slot of a row's pair and writes the other; padding rows sit
 * on the null slot 0).  A row breaks them when a slot of it lies outside
 * [0, N); when it is real (read slot not 0) and another real row has the same
 * read slot; or, for a twin write (write_slot not NULL), when it is real and
 * its write slot is its own read slot, is 0, or is another row's read or
 * write slot other than 0.  Enqueues one workgroup on `stream` (comparing
 * every pair of rows: O(B^2) work, for debugging, not for the hot loop) that
 * writes result[0] = the number of rows that break a precondition and
 * result[1] = the first of them, or -1; `result` is a caller-owned device
 * int32[2].  Stream-ordered, capturable, no allocation.  Uses dims' B and N.
 * B == 0 returns GDN_OK and enqueues nothing (result untouched);
 * GDN_ERR_NULL without read_slot or result.
 */
gdn_status gdn_check_slots(const gdn_dims *dims, const int32_t *read_slot, const int32_t *write_slot,
                           int32_t *result, hipStream_t stream);

/*
 * gdn_slot_reset -- zero slots of the pool (PR #1139, "Tests": rollback and
 * release zero both slots of a request).  For each i < n with
 * s = slots[i] in [1, N): state[s] (H_v*d_k*d_v fp32) and conv_state[s]
 * ((W-1)*C bf16) become +0.0.  Slot 0 and indices outside [1, N) are skipped
 * (the null slot is never written).  Uses dims' H_k, H_v, d_k, d_v, W and N
 * (B and T are ignored).  n = 0 returns GDN_OK at once; 0 <= n <= 65535.
 * Alignment: state 16 bytes, conv_state 8 bytes.
 */
gdn_status gdn_slot_reset(const gdn_dims *dims, float *state, gdn_bf16 *conv_state, const int32_t *slots,
                          int32_t n, hipStream_t stream);

/*
 * gdn_slot_copy -- copy whole slots (PR #1139, "Tests": decode snapshots and
 * forks must read the right slot; a prefix snapshot is the conv window and
 * the state).  For each i < n with src = src_slots[i] in [0, N) and
 * dst = dst_slots[i] in [1, N): state[dst] = state[src] and
 * conv_state[dst] = conv_state[src], bit for bit.  Pairs with dst = 0 or an
 * index out of range are skipped.  Preconditions (not checked): the
 * destinations are distinct and none is also a source in the same call.
 * Sizes and alignment as gdn_slot_reset.
 */
gdn_status gdn_slot_copy(const gdn_dims *dims, float *state, gdn_bf16 *conv_state, const int32_t *src_slots,
                         const int32_t *dst_slots, int32_t n, hipStream_t stream);

/* Static text for a status code (host only). */
const char *gdn_status_string(gdn_status status);

/*
 * gdn_traffic_probe -- calibration: the state traffic of gdn_decode_step at
 * the same shapes and slots, with no arithmetic, in one of several workgroup
 * designs (the method of PR #1139, "Numbers": a kernel with the step's reads
 * and writes and no math, and its read-only and write-only halves, gives the
 * practical ceiling of the step's traffic; several designs make that ceiling
 * the best of them rather than one kernel's).
 *
 * B rows x H heads of d_k x d_v fp32 tiles in state [N][H][d_k][d_v]:
 *   probe->traffic  0 read only (the read slots), 1 write only (the write
 *                   slots), 2 copy (read slot -> write slot: twin traffic),
 *                   3 read and write back (in-place traffic)
 *   probe->layout   0 the rows' slots: read_slot[r], write_slot[r] (rows with
 *                   a slot outside [1, N) move nothing);
 *                   1 consecutive slots: B slots from read_slot[0] on, written
 *                   to B slots from write_slot[0] on (the launch moves nothing
 *                   unless both ranges lie in [1, N))
 *   probe->shape    0, 1, 2: the fused step's thread layout (a wave holds the
 *                   eight row groups of 32 columns, 2 d_v threads a tile), 1,
 *                   2 or 4 whole tiles a workgroup (2 and 4: d_k = d_v = 128);
 *                   3: plain copy chunks of threads x loads x 16 bytes, as
 *                   set by the fields below (the tile must be a multiple of
 *                   the chunk);
 *                   4: an empty kernel (the launch floor);
 *                   5: one workgroup loads read_slot[0], then that slot's
 *                   first tile (the floor of a step's first dependent loads)
 *   probe->hold_ns  0, or: every workgroup holds its stores until this long
 *                   after it started (at most 1 ms), which puts the launch's
 *                   reads ahead of its writes when long enough; for
 *                   measurement only (not with a persistent grid)
 *   probe->order    0: each store goes as soon as its own load is in;
 *                   1: a lane's stores wait for all of its loads;
 *                   2: a workgroup's stores wait for all of its loads
 *                   (shapes 0-3)
 *   probe->threads  shape 3: workgroup size, 256, 512 or 1024
 *   probe->loads    shape 3: 16-byte loads a lane, 1, 4, 8 or 16, with
 *                   threads x loads at most 4096 (64 KiB a chunk)
 *   probe->persistent  shape 3: 0, one chunk a workgroup; k in 1..8, k
 *                   workgroups a compute unit walking the chunks in turn
 *   probe->policy   shapes 0-3: 0 streaming loads and stores (nt, as the
 *                   step's state accesses), 1 plain, 2 system scope (sc0 sc1)
 * sink [1] fp32 receives nothing in practice; it keeps read-only loads alive.
 * write_slot is required for traffic 1 and 2, ignored otherwise.  Statuses:
 * GDN_ERR_NULL, GDN_ERR_SHAPE (B < 0, H or N < 1, a value out of range, a
 * contiguous range over 2 GiB), GDN_ERR_UNSUPPORTED (head dims not 64/128, a
 * shape or chunk not built for them, misaligned state).
 */
typedef struct gdn_probe {
    int32_t traffic, layout, shape, hold_ns;
    int32_t order, threads, loads, persistent, policy;
} gdn_probe;

gdn_status gdn_traffic_probe(const gdn_probe *probe, int32_t B, int32_t H, int32_t d_k, int32_t d_v, int32_t N,
                             float *state, const int32_t *read_slot, const int32_t *write_slot, float *sink,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
