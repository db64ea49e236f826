/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for the Gated DeltaNet decode
 * step with a slot-addressed state pool.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded host arrays that
 * gdn_inputs.py draws.
 *
 * Sources (the mstar pull-request pages):
 *   - PR #1139, "Why" and "What changed": the GDN rule is the recurrent state
 *     update of a Qwen3.5 linear-attention layer; a request's state lives in
 *     a pooled slot; a decode step (one token a row) either reads one slot and
 *     writes the twin slot, which commit then swaps, or updates in place
 *     (keep_in_place); both give the same values.
 *   - PR #1139, "What changed": causal_conv1d_decode updates the conv window
 *     for one token a row and honours a separate write slot.
 *   - PR #1139, "Tests", and PR #965, "What changed": padding rows address
 *     the null slot 0 and never change a real row's result.
 *   - The update itself is the gated delta rule of Gated DeltaNet (Yang,
 *     Kautz, Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta
 *     Rule", ICLR 2025): decay the state by exp(g), correct it towards v along
 *     the normalised key with strength beta, read it out with the query.  The
 *     pages never print the equations; the statement order used here is:
 *     decay, predict with the decayed state, correct, read out the corrected
 *     state.
 *
 * Readings where the pages are silent (each also listed with the design notes):
 *   - state S of a value head is d_k x d_v, S[i][j] with i over keys; the
 *     correction is S[i][j] += beta * k[i] * (v[j] - sum_i' S[i'][j] k[i']),
 *     and the read-out is o[j] = sum_i S[i][j] q[i];
 *   - q and k are L2-normalised as x / sqrt(sum x^2 + eps); q is then scaled
 *     by q_scale;
 *   - the conv window holds the W-1 previous inputs of each channel, oldest
 *     first; the last tap multiplies the current token; SiLU follows the conv
 *     on every q/k/v channel;
 *   - channel order is q | k | v, head-major; value head hv reads key head
 *     hv / (H_v / H_k);
 *   - g (log decay) and beta arrive precomputed per (row, token, value head);
 *   - a row whose read slot is 0 is padding: its output is +0.0 and it reads
 *     and writes no slot; slot 0 is the null slot and never holds a row's
 *     state or window, so a real row that would write it is refused;
 *   - the state is held in fp64 during a call and rounded to fp32 (round to
 *     nearest even) only where it is stored back to the pool; conv-window
 *     values are bf16 inputs and are stored back exactly.
 *
 * Parity pins: every function here is checked in tests/test_oracle_pins.py
 * against closed forms, invariants, a library convolution and a brute-force
 * product-form recurrence (see that file's header for the list).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- storage conversions (exact where stated) ---------- */

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The value must already be a bf16 number (conv windows only ever hold bf16
 * inputs); returns -1 in *ok if it is not, so a caller can refuse. */
static uint16_t double_to_bf16_bits_exact(double d, int *ok)
{
    float f = (float)d;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0xFFFFu) != 0u || (double)f != d)
        *ok = 0;
    return (uint16_t)(u >> 16);
}

/* ---------- elementwise pieces ---------- */

/* SiLU (sigmoid-weighted linear unit): y * sigmoid(y). */
double oracle_silu(double y)
{
    return y / (1.0 + exp(-y));
}

/* out = x / sqrt(sum x^2 + eps) * scale, over n values. */
void oracle_l2norm(int n, const double *x, double eps, double scale, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double den = sqrt(ss + eps);
    for (int i = 0; i < n; ++i)
        out[i] = x[i] / den * scale;
}

/* ---------- conv decode (PR #1139, "What changed": causal_conv1d_decode) ----
 *
 * One token of one row, all C channels.  win is [W-1][C] (oldest first) and
 * is shifted in place: afterwards it holds the last W-1 inputs including
 * x_t.  y[c] = sum_w wgt[c][w] * [win, x_t][w] (+ bias[c]), then SiLU if
 * act != 0.
 */
void oracle_conv_token(int C, int W, const uint16_t *conv_w, const uint16_t *conv_b,
                       double *win, const uint16_t *x_t, int act, double *y)
{
    for (int c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int w = 0; w < W - 1; ++w)
            acc += bf16_bits_to_double(conv_w[(size_t)c * W + w]) * win[(size_t)w * C + c];
        double xc = bf16_bits_to_double(x_t[c]);
        acc += bf16_bits_to_double(conv_w[(size_t)c * W + (W - 1)]) * xc;
        if (conv_b)
            acc += bf16_bits_to_double(conv_b[c]);
        y[c] = act ? oracle_silu(acc) : acc;
        for (int w = 0; w + 1 < W - 1; ++w)
            win[(size_t)w * C + c] = win[(size_t)(w + 1) * C + c];
        if (W >= 2)
            win[(size_t)(W - 2) * C + c] = xc;
    }
}

/* Standalone pooled conv decode over B rows (the causal_conv1d_decode
 * contract): reads each row's window from conv_state[read_slot[r]], writes the
 * shifted window to conv_state[write_slot[r]] (read slot when write_slot is
 * NULL), y to out[r][c] in fp64.  Padding rows (read slot 0) give y = 0 and
 * touch no slot.  conv_state is [N][W-1][C] bf16 bits.  Returns 0, or -1 if a
 * slot is out of range, a real row's write slot is the null slot 0, or a
 * window value is not bf16. */
int oracle_conv_decode(int B, int C, int W, int N, const uint16_t *x, int64_t x_row_stride,
                       const uint16_t *conv_w, const uint16_t *conv_b, uint16_t *conv_state,
                       const int32_t *read_slot, const int32_t *write_slot, int act,
                       double *out)
{
    double *win = (double *)malloc(sizeof(double) * (size_t)(W - 1 > 0 ? W - 1 : 1) * C);
    int ok = 1;
    for (int r = 0; r < B && ok; ++r) {
        int rs = read_slot[r];
        int ws = write_slot ? write_slot[r] : rs;
        if (rs < 0 || rs >= N || ws < 0 || ws >= N) { ok = 0; break; }
        /* a real row never writes the null slot: slot 0 holds no row's window */
        if (rs != 0 && ws == 0) { ok = 0; break; }
        if (rs == 0) {
            for (int c = 0; c < C; ++c)
                out[(size_t)r * C + c] = 0.0;
            continue;
        }
        const uint16_t *src = conv_state + (size_t)rs * (W - 1) * C;
        for (size_t e = 0; e < (size_t)(W - 1) * C; ++e)
            win[e] = bf16_bits_to_double(src[e]);
        oracle_conv_token(C, W, conv_w, conv_b, win, x + (size_t)r * x_row_stride, act,
                          out + (size_t)r * C);
        uint16_t *dst = conv_state + (size_t)ws * (W - 1) * C;
        for (size_t e = 0; e < (size_t)(W - 1) * C; ++e)
            dst[e] = double_to_bf16_bits_exact(win[e], &ok);
    }
    free(win);
    return ok ? 0 : -1;
}

/* ---------- gated delta rule, one value head, one token ----------
 *
 * S is d_k x d_v row-major (S[i*d_v + j]), updated in place in fp64:
 *   alpha = exp(g);           S <- alpha * S
 *   pred[j] = sum_i S[i][j] k[i]
 *   S[i][j] <- S[i][j] + beta * k[i] * (v[j] - pred[j])
 *   o[j] = sum_i S[i][j] q[i]
 * q and k are passed already normalised (and q already scaled).
 */
void oracle_delta_rule(int dk, int dv, double *S, const double *q, const double *k,
                       const double *v, double g, double beta, double *o)
{
    double alpha = exp(g);
    double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= alpha;
    for (int j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i)
            s += S[(size_t)i * dv + j] * k[i];
        pred[j] = s;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] += beta * k[i] * (v[j] - pred[j]);
    for (int j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i)
            s += S[(size_t)i * dv + j] * q[i];
        o[j] = s;
    }
    free(pred);
}

/* ---------- one token of one row, every value head ----------
 *
 * Conv decode + SiLU over all C channels (the window advances by one token),
 * then for each value head hv: q and k of key head hv / (H_v / H_k), v of
 * head hv (channel order q | k | v, head-major), L2-normalised q (times
 * q_scale) and k, and the gated delta rule on that head's tile of S.
 * g_t, beta_t: [H_v] gates of this token; o_t: [H_v][d_v].  y, qh, kh are
 * work arrays of C, d_k and d_k doubles.
 */
static void oracle_row_token(int H_k, int H_v, int d_k, int d_v, int W, const uint16_t *x_t,
                             const uint16_t *conv_w, const uint16_t *conv_b, double *win, double *S,
                             const float *g_t, const float *beta_t, double *o_t, double q_scale, double l2_eps,
                             double *y, double *qh, double *kh)
{
    const int G = H_v / H_k;
    const int C = 2 * H_k * d_k + H_v * d_v;
    const size_t tile = (size_t)d_k * d_v;
    oracle_conv_token(C, W, conv_w, conv_b, win, x_t, 1, y);
    for (int hv = 0; hv < H_v; ++hv) {
        int hk = hv / G;
        const double *q = y + (size_t)hk * d_k;
        const double *k = y + (size_t)H_k * d_k + (size_t)hk * d_k;
        const double *v = y + (size_t)2 * H_k * d_k + (size_t)hv * d_v;
        oracle_l2norm(d_k, q, l2_eps, q_scale, qh);
        oracle_l2norm(d_k, k, l2_eps, 1.0, kh);
        oracle_delta_rule(d_k, d_v, S + (size_t)hv * tile, qh, kh, v, (double)g_t[hv], (double)beta_t[hv],
                          o_t + (size_t)hv * d_v);
    }
}

/* ---------- the whole decode step over a pooled state ----------
 *
 * Layouts (host arrays):
 *   x          [B][T][C] bf16 bits, row stride x_row_stride elements, C = 2*H_k*d_k + H_v*d_v
 *   conv_w     [C][W] bf16 bits;  conv_b [C] bf16 bits or NULL
 *   conv_state [N][W-1][C] bf16 bits
 *   state      [N][H_v][d_k][d_v] fp32
 *   g, beta    [B][T][H_v] fp32
 *   read_slot, write_slot [B] int32 (write_slot NULL => in place)
 *   out        [B][T][H_v][d_v] fp64 (unrounded read-out)
 * Rows are processed in order; a row's new state and window are stored to
 * its write slot after its last token.  Returns 0, or -1 on an invalid slot
 * (out of range, or a real twin row whose write slot is its read slot or the
 * null slot 0), shape or a non-bf16 window value.
 */
int oracle_gdn_decode_step(int B, int T, int H_k, int H_v, int d_k, int d_v, int W, int N,
                           const uint16_t *x, int64_t x_row_stride, const uint16_t *conv_w,
                           const uint16_t *conv_b, uint16_t *conv_state, float *state,
                           const float *g, const float *beta, const int32_t *read_slot,
                           const int32_t *write_slot, double *out, double q_scale, double l2_eps)
{
    if (H_k <= 0 || H_v % H_k != 0 || W < 1 || T < 1)
        return -1;
    const int C = 2 * H_k * d_k + H_v * d_v;
    const size_t tile = (size_t)d_k * d_v;
    const size_t slot_state = (size_t)H_v * tile;
    const size_t slot_conv = (size_t)(W - 1) * C;

    double *S = (double *)malloc(sizeof(double) * slot_state);
    double *win = (double *)malloc(sizeof(double) * (slot_conv ? slot_conv : 1));
    double *y = (double *)malloc(sizeof(double) * (size_t)C);
    double *qh = (double *)malloc(sizeof(double) * (size_t)d_k);
    double *kh = (double *)malloc(sizeof(double) * (size_t)d_k);
    int ok = 1;

    for (int r = 0; r < B && ok; ++r) {
        int rs = read_slot[r];
        int ws = write_slot ? write_slot[r] : rs;
        if (rs < 0 || rs >= N || ws < 0 || ws >= N) { ok = 0; break; }
        /* a real twin row writes a slot of its own other than the one it reads,
         * and never the null slot, which holds no row's state */
        if (write_slot && rs != 0 && (ws == 0 || ws == rs)) { ok = 0; break; }
        double *out_r = out + (size_t)r * T * H_v * d_v;
        if (rs == 0) {
            for (size_t e = 0; e < (size_t)T * H_v * d_v; ++e)
                out_r[e] = 0.0;
            continue;
        }
        const float *src = state + (size_t)rs * slot_state;
        for (size_t e = 0; e < slot_state; ++e)
            S[e] = (double)src[e];
        const uint16_t *csrc = conv_state + (size_t)rs * slot_conv;
        for (size_t e = 0; e < slot_conv; ++e)
            win[e] = bf16_bits_to_double(csrc[e]);

        for (int t = 0; t < T; ++t) {
            size_t rt = (size_t)r * T + t;
            oracle_row_token(H_k, H_v, d_k, d_v, W, x + (size_t)r * x_row_stride + (size_t)t * C, conv_w, conv_b,
                             win, S, g + rt * H_v, beta + rt * H_v, out_r + (size_t)t * H_v * d_v, q_scale, l2_eps,
                             y, qh, kh);
        }

        float *dst = state + (size_t)ws * slot_state;
        for (size_t e = 0; e < slot_state; ++e)
            dst[e] = (float)S[e];
        uint16_t *cdst = conv_state + (size_t)ws * slot_conv;
        for (size_t e = 0; e < slot_conv; ++e)
            cdst[e] = double_to_bf16_bits_exact(win[e], &ok);
    }

    free(S); free(win); free(y); free(qh); free(kh);
    return ok ? 0 : -1;
}

/* Commit of a twin-slot step: each row's read and write slot trade places, so
 * the next step reads what this one wrote (PR #1139, "What changed"). */
void oracle_slot_commit(int32_t *read_slot, int32_t *write_slot, int B)
{
    for (int r = 0; r < B; ++r) {
        int32_t t = read_slot[r];
        read_slot[r] = write_slot[r];
        write_slot[r] = t;
    }
}

/* ---------- slot lifecycle (PR #1139, "Tests": rollback and release zero both
 * slots of a request; decode snapshots and forks read the right slot) ----------
 *
 * A slot's contents are its state [H_v][d_k][d_v] fp32 and its conv window
 * [W-1][C] bf16.  Slot 0 is the null slot: it is never written.  A slot index
 * outside [0, N) is skipped.
 */
void oracle_slot_reset(int H_v, int d_k, int d_v, int W, int C, int N, float *state, uint16_t *conv_state,
                       const int32_t *slots, int n)
{
    const size_t slot_state = (size_t)H_v * d_k * d_v;
    const size_t slot_conv = (size_t)(W - 1) * C;
    for (int i = 0; i < n; ++i) {
        int s = slots[i];
        if (s <= 0 || s >= N)
            continue;
        for (size_t e = 0; e < slot_state; ++e)
            state[(size_t)s * slot_state + e] = 0.0f;
        for (size_t e = 0; e < slot_conv; ++e)
            conv_state[(size_t)s * slot_conv + e] = 0;
    }
}

/* dst[i] <- src[i] for every pair, contents taken as they were before the call
 * (the destinations must be distinct and must not be any pair's source). */
void oracle_slot_copy(int H_v, int d_k, int d_v, int W, int C, int N, float *state, uint16_t *conv_state,
                      const int32_t *src, const int32_t *dst, int n)
{
    const size_t slot_state = (size_t)H_v * d_k * d_v;
    const size_t slot_conv = (size_t)(W - 1) * C;
    for (int i = 0; i < n; ++i) {
        int a = src[i], b = dst[i];
        if (a < 0 || a >= N || b <= 0 || b >= N)
            continue;
        memcpy(state + (size_t)b * slot_state, state + (size_t)a * slot_state, slot_state * sizeof(float));
        memcpy(conv_state + (size_t)b * slot_conv, conv_state + (size_t)a * slot_conv, slot_conv * sizeof(uint16_t));
    }
}

/* ---------- a state per token (PR #1139, "What changed": speculative
 * decoding keeps a state per token in its slots) ----------
 *
 * Like oracle_gdn_decode_step in place over T tokens, except that after token
 * t the state and the conv window are stored (fp32 / exact bf16) to slot
 * token_slots[r*T + t] when that slot is not 0, and nothing is stored at the
 * end.  The state stays fp64 between tokens; each stored copy is rounded to
 * fp32.  A row with read slot 0 is padding (zero output, no slot touched).
 * Returns 0, or -1 on an invalid slot.
 */
int oracle_gdn_decode_step_tokens(int B, int T, int H_k, int H_v, int d_k, int d_v, int W, int N,
                                  const uint16_t *x, int64_t x_row_stride, const uint16_t *conv_w,
                                  const uint16_t *conv_b, uint16_t *conv_state, float *state,
                                  const float *g, const float *beta, const int32_t *read_slot,
                                  const int32_t *token_slots, double *out, double q_scale, double l2_eps)
{
    if (H_k <= 0 || H_v % H_k != 0 || W < 2 || T < 1)
        return -1;
    const int C = 2 * H_k * d_k + H_v * d_v;
    const size_t tile = (size_t)d_k * d_v;
    const size_t slot_state = (size_t)H_v * tile;
    const size_t slot_conv = (size_t)(W - 1) * C;
    double *S = (double *)malloc(sizeof(double) * slot_state);
    double *win = (double *)malloc(sizeof(double) * slot_conv);
    double *y = (double *)malloc(sizeof(double) * (size_t)C);
    double *qh = (double *)malloc(sizeof(double) * (size_t)d_k);
    double *kh = (double *)malloc(sizeof(double) * (size_t)d_k);
    int ok = 1;
    for (int r = 0; r < B && ok; ++r) {
        int rs = read_slot[r];
        if (rs < 0 || rs >= N) { ok = 0; break; }
        for (int t = 0; t < T; ++t) {
            int ts = token_slots[(size_t)r * T + t];
            if (ts < 0 || ts >= N) ok = 0;
        }
        if (!ok)
            break;
        double *out_r = out + (size_t)r * T * H_v * d_v;
        const int padding = (rs == 0);
        if (padding) {
            memset(out_r, 0, sizeof(double) * (size_t)T * H_v * d_v);
            continue;
        }
        for (size_t e = 0; e < slot_state; ++e)
            S[e] = (double)state[(size_t)rs * slot_state + e];
        for (size_t e = 0; e < slot_conv; ++e)
            win[e] = bf16_bits_to_double(conv_state[(size_t)rs * slot_conv + e]);
        for (int t = 0; t < T; ++t) {
            size_t rt = (size_t)r * T + t;
            oracle_row_token(H_k, H_v, d_k, d_v, W, x + (size_t)r * x_row_stride + (size_t)t * C, conv_w, conv_b,
                             win, S, g + rt * H_v, beta + rt * H_v, out_r + (size_t)t * H_v * d_v, q_scale, l2_eps,
                             y, qh, kh);
            int ts = token_slots[(size_t)r * T + t];
            if (ts != 0) {
                for (size_t e = 0; e < slot_state; ++e)
                    state[(size_t)ts * slot_state + e] = (float)S[e];
                for (size_t e = 0; e < slot_conv; ++e)
                    conv_state[(size_t)ts * slot_conv + e] = double_to_bf16_bits_exact(win[e], &ok);
            }
        }
    }
    free(S); free(win); free(y); free(qh); free(kh);
    return ok ? 0 : -1;
}
