/*
 * spec_verify.h -- batched speculative-decoding verification on one AMD
 * MI355X (gfx950) GPU, behind a plain C ABI.
 *
 * What one call computes, per sequence b of a batch of B (sources are cited
 * by page title and section):
 *
 *   - target logits at K+1 positions and draft logits at K positions over a
 *     vocabulary of V tokens are turned into sampling laws p_i and q_i by a
 *     temperature softmax ("Speculative Decoding: Draft, Verify, and Correct",
 *     section "Preserve the distribution you actually intend"; "Speculative
 *     decoding: why correcting a rejection is not resampling from the target",
 *     section 1);
 *   - drafted tokens d_0..d_{K-1} are tested in order, each kept with
 *     probability min(1, p_i(d_i)/q_i(d_i)), until the first rejection j
 *     ("Draft, Verify, and Correct", sections "Name the two distributions at
 *     one prefix" and "Verify several proposed tokens in one target pass");
 *   - at j < K a correction is drawn from the normalised positive residual
 *     [p_j - q_j]_+ ("Draft, Verify, and Correct", section "Why the correction
 *     recovers the target"; "... not resampling from the target", sections 2
 *     and 3); at j = K a bonus token is drawn from p_K ("... not resampling
 *     from the target", section 5);
 *   - greedy mode keeps a draft iff it is the target argmax and emits the
 *     argmax otherwise ("Speculative Decoding: How a Small Model Speeds Up a
 *     Big One Without Changing Its Output", section "The Guarantee Behind
 *     Rejection Sampling"); margin mode also keeps a mismatched draft when
 *     p(d)/p(argmax) exceeds tau ("Margins, Not Windows: Training-Free
 *     Per-Step Lossy Speculative Decoding", section 3, margin-based lossy
 *     verification);
 *   - the accepted-length histogram of the call and a per-slot rolling
 *     acceptance EMA are maintained ("... not resampling from the target",
 *     section 7; "Margins, Not Windows", section 3, dynamic tree shaping).
 *
 * Short names used for these pages further down:
 *   [DVC]   "Speculative Decoding: Draft, Verify, and Correct"
 *   [SMB]   "Speculative Decoding: How a Small Model Speeds Up a Big One
 *            Without Changing Its Output"
 *   [RNR]   "Speculative decoding: why correcting a rejection is not
 *            resampling from the target"
 *   [MNW]   "Margins, Not Windows: Training-Free Per-Step Lossy Speculative
 *            Decoding"
 *   [DRIFT] "Speculative Decoding Under Distribution Shift: DRIFT
 *            Recalibration"
 *
 * Conventions fixed by this library where the pages leave a choice:
 *   - u[b][i] decides position i (keep iff p >= q or u < p/q, strict);
 *     u[b][K] drives the one correction/bonus draw (inverse CDF in index
 *     order: smallest v whose inclusive prefix weight exceeds u times the
 *     total; clamped to the last positive-weight token). Greedy and margin
 *     modes read no uniforms.
 *   - argmax ties go to the lowest index, on raw logit values.
 *   - q(d) = 0 keeps the draft (counted); Z = 0 after a rejection (rounding
 *     only) draws from p_j instead (counted).
 *   - a sequence whose drafted token is outside [0, V), or whose needed logit
 *     row holds NaN or +inf or only -inf, is reported invalid: accept_len -1,
 *     all tokens -1, not counted in the histogram, EMA untouched. Needed rows:
 *     all K+1 target rows, plus all K draft rows in stochastic mode.
 *   - logits times log2(e)/T must be finite in fp32; rows that overflow are
 *     reported invalid.
 *
 * Threading and streams: every call is asynchronous on the stream it is
 * given, never allocates, never synchronises and never touches the default
 * stream, so it may be captured into a HIP graph. Calls on one handle must be
 * ordered (one stream, or explicit events); the handle's workspace and EMA
 * state are shared by all of them.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify_handle spec_verify_handle;

enum { SV_DTYPE_F32 = 0, SV_DTYPE_BF16 = 1 };
enum { SV_MODE_STOCHASTIC = 0, SV_MODE_GREEDY = 1, SV_MODE_MARGIN = 2 };
enum {
    SV_OK = 0,
    SV_EINVAL = -1,        /* bad argument; nothing was enqueued */
    SV_EUNSUPPORTED = -2,  /* unknown dtype */
    SV_ENOMEM = -3,        /* device allocation failed (init, set_residual) */
    SV_EHIP = -4           /* a HIP call or launch failed; see spec_verify_last_error */
};

/* Device-side counters, cumulative since init or the last reset. */
typedef struct spec_verify_stats {
    uint64_t sequences;        /* valid sequences verified */
    uint64_t invalid;          /* sequences reported invalid (bad token or row) */
    uint64_t zero_q_accepts;   /* kept drafts whose draft probability was 0 */
    uint64_t z0_fallbacks;     /* rejections whose residual summed to 0 */
    uint64_t calls;            /* successful spec_verify calls (host counter) */
} spec_verify_stats;

/*
 * Create a handle for batches of up to max_batch sequences with K drafts over
 * a vocabulary of V tokens stored as logits_dtype (SV_DTYPE_F32 or
 * SV_DTYPE_BF16). 1 <= K <= 63, 1 <= V < 2^31 / (K+1), 1 <= max_batch.
 * ema_decay in [0, 1] weights the previous EMA value. Uses the current HIP
 * device; the handle owns its device workspace (about 64 * max_batch * K
 * bytes plus a few KB per sequence), the EMA state (float64 value and int32
 * count per slot) and the counters, and frees them in spec_verify_destroy.
 * Synchronises the device once (initialisation only).
 *
 * Path selection and tuning are read from the environment here (for tests and
 * measurement; the defaults are the tuned ones):
 *   SPEC_VERIFY_TARGET_WGS       streaming-pass workgroups to aim for (2048)
 *   SPEC_VERIFY_TARGET_WGS_MAX   the same for the argmax pass of greedy and
 *                                margin calls (6144)
 *   SPEC_VERIFY_NSEG             fixed segments per row (0 = from the target)
 *   SPEC_VERIFY_FINISH_SEQ       0: stochastic draw as separate scan, tile-sum
 *                                and pick kernels instead of one workgroup per
 *                                sequence (that path is always used when a row
 *                                has more than 256 draw tiles)
 *   SPEC_VERIFY_TILES_PER_GROUP  draw tiles per workgroup on that path (16)
 *   SPEC_VERIFY_CLAIM_TILES      0: the per-sequence finish gives wavefront w
 *                                the draw tiles w, w + 16, ... instead of
 *                                each wavefront claiming the next tile from a
 *                                counter in LDS (1)
 *   SPEC_VERIFY_FUSED_MIN_B      smallest batch that streams and finishes each
 *                                sequence in one kernel (0 = never)
 *   SPEC_VERIFY_TRUNC32_LIST     0: float32 truncation without the one-read
 *                                top-k list pass (1)
 *   SPEC_VERIFY_TRUNC32_BUF      0: float32 truncation narrows every row by
 *                                digit reads, never through an LDS copy (1)
 *   SPEC_VERIFY_TRUNC32_ONE      0: float32 rows the list pass hands over
 *                                (top-p alone, top-k past its lists or tied)
 *                                skip the one-read pass that follows it (1)
 *   SPEC_VERIFY_MERGE_IN_FINISH  0: the residual side output's candidate
 *                                lists are merged by a kernel of their own
 *                                after the call instead of inside the
 *                                per-sequence finish (1)
 */
int spec_verify_init(spec_verify_handle **h, int max_batch, int K, int V,
                     int logits_dtype, double ema_decay);

/*
 * Verify B sequences (1 <= B <= max_batch). All pointers are device pointers
 * to contiguous row-major arrays, owned by the caller, aligned to their
 * element size; 16-byte alignment of the logit arrays (with V a multiple of 8
 * for bf16, 4 for fp32) selects the 128-bit load path.
 *
 *   target_logits   [B][K+1][V] logits_dtype
 *   draft_logits    [B][K][V]   logits_dtype; stochastic mode only (may be NULL otherwise)
 *   draft_tokens    [B][K]      int32
 *   uniforms        [B][K+1]    float32 in [0, 1); stochastic mode only (may be NULL otherwise)
 *   temperature     T > 0, finite (stochastic and margin modes; ignored by greedy)
 *   mode            SV_MODE_*
 *   tau             margin threshold (margin mode; finite), ignored otherwise
 *   out_tokens      [B][K+1]    int32: kept drafts, then the correction/bonus, then -1
 *   out_accept_len  [B]         int32: kept drafts j in 0..K (emitted = j+1); -1 if invalid
 *   out_accept_hist [K+1]       uint32: zeroed, then hist[j] counts this call's valid sequences
 *                               (the Python binding hands it out as an int32 tensor holding
 *                               these bits; counts stay below 2^31 for any B it accepts)
 *   stream          HIP stream the work is ordered on
 *
 * EMA slot b is updated with x = accept_len/K for every valid sequence b
 * (accept_len/k_b under the stopping rules of spec_verify_set_stops).
 * Returns SV_OK once the work is enqueued, or an error code with nothing
 * enqueued (SV_EINVAL for a NULL handle or required pointer, B out of range,
 * an unknown mode, T not finite or T <= 0 in stochastic/margin mode, tau not
 * finite in margin mode; SV_EHIP for a failed launch).
 */
int spec_verify(spec_verify_handle *h, int B,
                const void *target_logits, const void *draft_logits,
                const int32_t *draft_tokens, const float *uniforms,
                float temperature, int mode, float tau,
                int32_t *out_tokens, int32_t *out_accept_len,
                uint32_t *out_accept_hist, hipStream_t stream);

/* Free everything the handle owns (synchronises the device). NULL-safe. */
int spec_verify_destroy(spec_verify_handle *h);

/*
 * Optional per-call side outputs written by later spec_verify calls (device
 * pointers sized for max_batch; NULL disables each one):
 *   p_d    [B][K] float64: stochastic p_i(d_i); margin p_i(d_i)/p_i(argmax_i); greedy NaN
 *   q_d    [B][K] float64: stochastic q_i(d_i); NaN otherwise
 *   z      [B]    float64: residual total Z at the rejection (stochastic, j < K), else -1
 *   argmax [B][K+1] int32: lowest-index argmax of each target row (greedy and margin;
 *          -1 for rows past the draft count k_b of spec_verify_set_stops)
 * Values at positions after the first rejection are still filled. Invalid
 * sequences get NaN / -1.
 */
int spec_verify_set_aux(spec_verify_handle *h, double *p_d, double *q_d,
                        double *z, int32_t *argmax);

/*
 * Stopping rules for later spec_verify calls on this handle ([DVC] "Verify
 * several proposed tokens in one target pass" and "Speculation needs cache
 * rollback": end-of-sequence and length limits can end a cycle before its
 * draft block is used up, and the returned tokens must agree with them).
 *
 *   eos_token  end-of-sequence token id, or -1 for none (< -1: SV_EINVAL)
 *   draft_len  [max_batch] int32 device array, k_b in [0, K]: drafts tested
 *              for sequence b; NULL = K for every sequence
 *   max_emit   [max_batch] int32 device array, m_b >= 1: tokens sequence b
 *              may emit in this cycle; NULL = no limit
 *
 * Per sequence the walk tests positions 0..k_b-1 (j = first rejection, else
 * k_b; the bonus comes from target row k_b); the emission d_0..d_{j-1}, c is
 * cut after its first end-of-sequence token and to its first m_b tokens;
 * out_accept_len and the histogram count the drafts emitted; the correction
 * or bonus is drawn (with uniforms[b][K]) only when it is emitted, and z is
 * then -1. Only target rows 0..k_b and draft rows 0..k_b-1 are needed. A k_b
 * outside [0, K] or an m_b < 1 makes the sequence invalid. The arrays are
 * read by the device during later calls and stay owned by the caller; they
 * must outlive those calls. spec_verify_set_stops(h, -1, NULL, NULL) restores
 * the plain cycle.
 */
int spec_verify_set_stops(spec_verify_handle *h, int eos_token, const int32_t *draft_len,
                          const int32_t *max_emit);

/*
 * Top-k / top-p truncation for later stochastic spec_verify calls on this
 * handle ([RNR] s.1: p and q are the distributions the samplers really use,
 * after temperature and truncation; s.2: a mask that only the correction
 * sees breaks the guarantee). Every needed target and draft row of sequence
 * b is truncated with the same rules before the acceptance ratio, the
 * residual and the bonus draw use it:
 *
 *   top_k  [max_batch] int32 device array: keep the values at or above the
 *          top_k-th largest logit of the row, counted with multiplicity (all
 *          values tied with it stay); <= 0 or >= V: no top-k; NULL: off
 *   top_p  [max_batch] float32 device array: then keep, from the top, whole
 *          value levels up to and including the first level at which the
 *          kept mass reaches top_p of the top-k mass; >= 1: no top-p; not
 *          > 0 (or NaN): the sequence is invalid; NULL: off
 *
 * Kept tokens are renormalised, dropped ones have probability exactly 0.
 * Greedy and margin calls ignore the settings. bf16 and float32 logits are
 * supported, with V up to 524288 (bf16) or 262144 (float32) when V is a
 * multiple of 8 (bf16) or 4 (float32) and the logit tensors are 16-byte
 * aligned, else 65536 (larger V: spec_verify returns SV_EUNSUPPORTED). A
 * float32 call reads a needed row once when its top k + 1 values (k <= 383)
 * settle it, else two to six times (the k-th largest value and the top-p
 * level are narrowed 12, 10 and 10 bits of the value's order key at a time);
 * its normalisers carry a relative error below 1e-8 beyond the terms' own.
 * The arrays are read by
 * the device during later calls and stay owned by the caller; they must
 * outlive those calls. spec_verify_set_truncation(h, NULL, NULL) turns
 * truncation off. Returns SV_EINVAL for a NULL handle or a misaligned array.
 */
int spec_verify_set_truncation(spec_verify_handle *h, const int32_t *top_k,
                               const float *top_p);

/*
 * Tree-shape policy epilogue for later spec_verify calls on this handle
 * ([MNW] s.3, dynamic draft tree-shaping: a draft confidence score combines
 * the draft's top-1 probability with the rolling acceptance history and picks
 * the next step's (nsteps, top-k, ndt) between (3, 4, 4) and (7, 1, 8); five
 * consecutive zero-accept steps restore the starting configuration). After
 * each sequence's EMA update (the rolling acceptance; [MNW]'s alpha = 0.3 is
 * ema_decay = 0.7 at spec_verify_init):
 *
 *   DCS_b = min(1, draft_conf[b] * ema_b / d)   (ema_b = 0 before the first
 *                                                observation of slot b)
 *   shape = (3 + 4 DCS, 4 - 3 DCS, 4 + 4 DCS), each rounded half up;
 *   after five consecutive calls with accept_len = 0 (and k_b > 0) the slot's
 *   EMA restarts and the shape is (3, 4, 4).
 *
 * The pages give neither the combination nor d; this product is the reading
 * taken. Arguments (device pointers sized for max_batch, caller-owned, read
 * or written during later calls):
 *   draft_conf  [max_batch] float32: the draft's top-1 probability for this
 *               cycle, in [0, 1]; NULL turns the policy off
 *   d           saturation divisor, finite and > 0
 *   out_shape   [max_batch][3] int32: nsteps, top-k, ndt for the next step;
 *               (-1, -1, -1) for invalid sequences or draft_conf outside
 *               [0, 1], whose state is left alone
 *   out_dcs     [max_batch] float64 score, or NULL
 * The zero-accept streaks live in the handle; spec_verify_reset_ema clears
 * them with the EMA. Returns SV_EINVAL for a NULL handle, a NULL out_shape
 * with draft_conf set, a bad d or a misaligned array.
 */
int spec_verify_set_policy(spec_verify_handle *h, const float *draft_conf, double d,
                           int32_t *out_shape, double *out_dcs);

/*
 * Draft residual side output for later stochastic spec_verify calls
 * ([DRIFT] "The update rule and its objective": at every drafted position
 * both distributions are restricted to a shared top-m support, and the
 * target log-probability minus the draft log-probability there is the
 * supervision a draft recalibration memory learns from; m = 32 in its
 * ablations). For each valid sequence b and drafted position i < k_b:
 *
 *   S = the m tokens with the largest draft logits at position i (ties to
 *       the lower token index; all V tokens when V < m), listed by
 *       descending draft logit, then ascending index;
 *   out_support[b][i][s] = the s-th token of S;
 *   out_residual[b][i][s] = (x_t(v) - x_d(v)) / T - LSE_S(x_t / T) + LSE_S(x_d / T)
 *                         = log p_S(v) - log q_S(v), both laws renormalised on S.
 *
 * "Shared top m" is read as the draft's top m. Positions i >= k_b, invalid
 * sequences and slots s >= V hold -1 and NaN. Arrays are device pointers of
 * [max_batch][K][m] entries (int32 and float64), caller-owned, written by
 * later calls on their stream, by the call's own kernels or one kernel after
 * them. Where the call's streaming pass reads 16-byte chunks (bf16 or fp32
 * rows), that pass also keeps the draft rows' top-m candidates, and the
 * per-sequence finish merges them (or, when they do not fit beside it, one
 * small kernel after the call); otherwise (truncation, one kernel per
 * sequence, rows not in 16-byte chunks) one extra kernel reads each draft
 * row once more.
 * The first call with out_support set allocates the candidate lists,
 * max_batch * K * 32 KiB on the handle's device, kept until
 * spec_verify_destroy (SV_ENOMEM if that fails); spec_verify itself still
 * allocates nothing. bf16 and fp32 logits; 1 <= m <= 64 (else
 * SV_EINVAL). out_support = NULL turns it off.
 */
int spec_verify_set_residual(spec_verify_handle *h, int m, int32_t *out_support,
                             double *out_residual);

/*
 * Walk-order reading for later spec_verify calls: stochastic calls (also
 * with top-k / top-p truncation) and greedy and margin calls
 * ([DVC] "Verify several proposed tokens in one target pass": at the first
 * rejection the correction is drawn and later proposals are discarded;
 * [SMB] "Seeing It in Code": the walk over the drafts stops at the first
 * disagreement). on = 1: the rows of drafted position i (target row i, and
 * draft row i for stochastic calls) are read only when the walk reaches
 * position i, i.e. once positions 0..i-1 are kept, and nothing past the
 * first rejection is read (target row k_b, the bonus row, only when every
 * position is kept). The streaming, truncation (both passes) or argmax pass
 * then reads position 0's rows of every sequence, lists the sequences whose
 * walk keeps position 0 (the same test as the scan, from the partials), and
 * reads their remaining rows; the finish reads no further than the walk.
 * Rows of positions past the first rejection after position 0 may still be
 * read (not checked, and never used).
 * What changes for the caller, and only this: a sequence is invalid only when
 * a drafted token or a row that the walk reads is unusable (NaN, +inf or no
 * finite maximum), not when one past its first rejection is; p(d) and q(d),
 * or the margin ratio (spec_verify_set_aux), are NaN past the first
 * rejection, and the per-row argmax is -1 past it. End-of-sequence and
 * budget stops cut the emission, not the reading; top_p <= 0 or NaN still
 * makes a sequence invalid. Every other output equals that of the full
 * reading on the same inputs. Stochastic calls with the draft residual side
 * output read every row as usual.
 * on = 0 (the default) reads every needed row.
 * Returns SV_EINVAL for a NULL handle or on outside {0, 1}.
 */
int spec_verify_set_walk_order(spec_verify_handle *h, int on);

/* EMA state accessors, ordered on `stream`. Device pointers of max_batch entries. */
int spec_verify_get_ema(spec_verify_handle *h, double *ema_dev, int32_t *steps_dev,
                        hipStream_t stream);
int spec_verify_set_ema(spec_verify_handle *h, const double *ema_dev,
                        const int32_t *steps_dev, hipStream_t stream);
int spec_verify_reset_ema(spec_verify_handle *h, hipStream_t stream);

/* Copy the counters to host memory; synchronises `stream`. reset != 0 clears them. */
int spec_verify_get_stats(spec_verify_handle *h, spec_verify_stats *out, int reset,
                          hipStream_t stream);

/*
 * Profiling. With enable != 0, each later spec_verify call records HIP events
 * on its stream just before and just after its streaming pass over the logits
 * (with truncation: the window pass of the truncation passes) (up to 4096
 * calls between reads; later calls are not recorded), and with
 * bit 1 of enable set (enable = 2 or 3) also after its last kernel. The events
 * are timing-only (no system-scope fence) and created here, never in
 * spec_verify. spec_verify_profile_read waits for the recorded calls to finish
 * and returns the summed milliseconds of the streaming pass and of whole calls
 * (0 unless call ends are recorded), and how many calls were recorded, then
 * starts a new window. enable = 0 frees them.
 */
int spec_verify_profile(spec_verify_handle *h, int enable);
int spec_verify_profile_read(spec_verify_handle *h, double *stream_pass_ms, double *call_ms,
                             int *n_calls);

/*
 * Text of the last error on this handle ("" if none). Valid until the next
 * call. With h = NULL: the text of this thread's last failed
 * spec_verify_noalloc call, or "null handle" if there was none.
 */
const char *spec_verify_last_error(const spec_verify_handle *h);

/*
 * One verification without a handle and without any allocation, for callers
 * that cannot allocate device memory: code being captured into a HIP graph,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments and
 * outputs as spec_verify, with the handle's fixed sizes given per call
 * (K in 1..63, V >= 1, V * (K+1) < 2^31, B >= 1, logits_dtype SV_DTYPE_*),
 * on the current HIP device.
 *
 * The workspace (row partials, counters, the per-call EMA) lies in a 1 MiB
 * device array inside this library, one copy per GPU, held until the process
 * ends; its device address is looked up once per device on the first call
 * there. Nothing else is kept between calls: the EMA and the counters are not
 * maintained, and the optional side outputs, stopping rules, truncation,
 * policy and residual of a handle do not exist here. Every call on one GPU
 * uses the same array, so calls that overlap on one GPU (concurrent streams,
 * threads) race and must be ordered by the caller.
 *
 * Routes: the streaming pass then one workgroup per sequence (stochastic,
 * V <= 524288 for bf16 / 262144 for fp32 logit arrays in 16-byte chunks,
 * V <= 65536 otherwise), the argmax pass then the scan (greedy, margin).
 * Returns SV_OK once enqueued; SV_EINVAL, with nothing enqueued, for the
 * argument errors of spec_verify or when B * rows * segments of row partials
 * would not fit in the array (about B * (2K+1) * 24 bytes for large batches:
 * B = 1024 at K = 4 fits, B = 4096 at K = 7 does not); SV_EUNSUPPORTED for
 * V beyond the stochastic route's limit or an unknown dtype; SV_EHIP when the
 * array's address cannot be found or a launch fails. The message is read
 * with spec_verify_last_error(NULL).
 */
int spec_verify_noalloc(int B, int K, int V, int logits_dtype,
                        const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, const float *uniforms,
                        float temperature, int mode, float tau,
                        int32_t *out_tokens, int32_t *out_accept_len,
                        uint32_t *out_accept_hist, hipStream_t stream);

/* Library version string. */
const char *spec_verify_version(void);

/*
 * Measurement aid (no handle): one plain streaming read of `bytes` bytes at
 * device pointer `buf`, with the streaming pass's access pattern (256-thread
 * workgroups over 256.5 KB spans, 128-bit non-temporal loads), enqueued on
 * `stream`. It gives the achievable read bandwidth that the streaming pass is
 * compared with. buf must be 16-byte aligned and bytes a positive multiple of
 * 16 (else SV_EINVAL); sink is a device uint32 the kernel may write. SV_EHIP
 * if the launch fails.
 */
int spec_verify_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
