/*
 * topth.h -- C ABI of libtopth, Top-theta attention for AMD Instinct MI355X
 * (gfx950).
 *
 * Method: "Top-Theta Attention: Sparsifying Transformers by Compensated
 * Thresholding" (arXiv 2502.08363).  Each attention row keeps the post-softmax
 * elements s_j >= theta[head][row], where theta is a static threshold that
 * calibration sets to the mean, over calibration sequences, of the row's k-th
 * largest post-softmax value (Sec. 3.1, Algorithm 1, post-softmax variant).
 * Kept elements keep their full softmax denominator (exact SDC, Sec. 3.2.1,
 * Eq. 4) and the discarded mass beta is added back times the mean V row
 * (VMC, Sec. 3.2.2, Eq. 5-7).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" point to GPU memory of the current HIP device;
 *    pointers marked "host" point to CPU memory read before the call returns.
 *    The caller owns every buffer; the library allocates no device memory and
 *    keeps no state between calls except what it leaves in the caller's
 *    workspace (see "Workspace").
 *  - Tensors are dense, row-major, head dimension fastest:
 *      Q [B][Hq][L][d], K and V [B][Hkv][L][d] (decode caches [B][Hkv][Lmax][d]).
 *  - GQA: query head h reads KV head h / (Hq / Hkv); Hq must be a multiple of
 *    Hkv (Sec. 2.2 and 4.6 of the paper).  Every head keeps its own selection.
 *  - Element type: TOPTH_F32 (float) or TOPTH_BF16 (bfloat16) for Q, K, V and
 *    the attention output; scores, softmax statistics and accumulation are
 *    float32.  d must be 64 or 128.
 *  - scale: the positive score scale, normally 1/sqrt(d).
 *  - Row id: query position p, 0-based; a decode step with n cached keys (the
 *    current token included) is row n - 1.  Rows at or past n_rows of a
 *    theta slab use the slab's last row.
 *  - theta slab of one layer: float theta[Hq][n_rows], post-softmax
 *    probabilities; -INFINITY (or any value <= 0) keeps every element.
 *  - stream: a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; nothing synchronises the host.
 *  - Errors: argument errors return a negative status before any GPU work
 *    is enqueued; a failed launch returns TOPTH_EHIP.  No C++ exception
 *    crosses this interface.  A decode call that returns TOPTH_OK has been
 *    enqueued; whether its cross-workgroup exchange completed on the GPU is
 *    reported afterwards in the workspace (see "Workspace").
 *  - Threads and global state: any host thread may call any entry point.  The
 *    library's only process-wide state is a per-device cache of device
 *    properties (CU count, resident workgroups per kernel), filled on first
 *    use and never changed afterwards.
 *  - GPU sharing: the key chunks of one decode call wait for each other, so a
 *    decode call assumes that all of its workgroups are resident at once; it
 *    sizes its grid to the whole GPU.  Run it with the GPU's compute units to
 *    itself: work on other streams that holds compute units while a decode
 *    call runs (another decode call included) can delay some of its chunks
 *    past the bounded wait, and the affected groups then report poisoned
 *    outputs (never silently wrong ones).
 *
 * Workspace
 * ---------
 *  Decode and calibration (and prefill with VMC) need a device workspace of
 *  at least topth_workspace_size(...) bytes.  Calibration and prefill use it
 *  as plain scratch.  Decode keeps a header of TOPTH_WS_HEADER_BYTES (32-bit
 *  word 0: the status, word 1: the spin limit) and, after it, the slots
 *  through which the key chunks of one (batch, KV head) exchange partial
 *  results.  A decode workspace must be prepared by topth_workspace_init
 *  before its first use; a decode call whose exchange completes leaves it
 *  prepared again, so it serves any later decode call of any size up to its
 *  capacity.  A workspace that a calibration or prefill call has used must be
 *  prepared again before a decode call.  Two calls that overlap in time must
 *  not share a workspace.
 *
 *  Exchange failures.  Every wait of the exchange is bounded (by default
 *  about 4M polls of some 64 clocks each, about 0.1 s).  When one gives up,
 *  the kernel still runs to its end, and
 *    - the status word gets bit TOPTH_STATUS_EXCHANGE_TIMEOUT;
 *    - every output of each (batch, KV head) group whose exchange did not
 *      complete is poisoned: out and beta NaN, kept_count and vrows_read -1
 *      (kept_mask entries are unspecified);
 *    - slots may be left filled, so the workspace is no longer prepared:
 *      while the status word is nonzero, every later decode call on it
 *      poisons all of its outputs without reading the slots, until
 *      topth_workspace_init prepares it again.
 *  The running mean of topth_decode_append is updated in every case.  Read
 *  the status with topth_workspace_status.
 */
#ifndef TOPTH_H
#define TOPTH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TOPTH_OK = 0,
    TOPTH_EINVAL = -1,        /* NULL pointer, bad size or inconsistent shape   */
    TOPTH_EUNSUPPORTED = -2,  /* valid but not implemented (d, dtype, g, size)  */
    TOPTH_EWORKSPACE = -3,    /* workspace NULL or smaller than required        */
    TOPTH_EHIP = -4,          /* a HIP runtime call or kernel launch failed     */
    TOPTH_ESCRATCH = -5       /* topth_decode_noalloc: the shape needs more than
                                 its static scratch (TOPTH_NOALLOC_SCRATCH_BYTES) */
} topth_status;

typedef enum { TOPTH_F32 = 0, TOPTH_BF16 = 1 } topth_dtype;

/* flags of topth_prefill / topth_decode (and of the _pre calls below) */
#define TOPTH_VMC       0x1u  /* add beta * mu, mu = mean V row (Sec. 3.2.2, Eq. 7)     */
#define TOPTH_SDC_NONE  0x2u  /* divide kept weights by the kept mass only (softmax
                                 over the kept set) instead of exact SDC; beta = 0       */
/* estimates of the discarded softmax mass E~, pre-softmax calls only (Sec. 3.2.1);
   with none of TOPTH_SDC_NONE / _EXPTH / _OFFLINE set, E~ is the exact E      */
#define TOPTH_SDC_EXPTH   0x4u  /* exp-threshold: E~ = gamma (n - k~) exp(theta - max a) */
#define TOPTH_SDC_OFFLINE 0x8u  /* offline-calibrated: E~ = e_tilde[h][row]              */
/* output format of every prefill and decode call: with TOPTH_BF16 inputs, out
   is float32 (the float32 result before any bfloat16 rounding) instead of
   bfloat16, same shape; with TOPTH_F32 inputs out is float32 either way      */
#define TOPTH_OUT_F32     0x10u

/* op codes of topth_workspace_size */
#define TOPTH_OP_CALIBRATE 0
#define TOPTH_OP_PREFILL   1
#define TOPTH_OP_DECODE    2
#define TOPTH_OP_CALIBRATE_PRE_E 3   /* topth_calibrate_pre with esum != NULL */
#define TOPTH_OP_CALIBRATE_MKC 4     /* topth_calibrate_mkc */

#define TOPTH_WS_HEADER_BYTES 65536
#define TOPTH_STATUS_EXCHANGE_TIMEOUT 0x1   /* bit of the workspace status word */
#define TOPTH_MAX_NK 8        /* most k values one calibration call can target */
#define TOPTH_MKC_MAX_TARGETS 64     /* most k values one topth_calibrate_mkc call returns */
#define TOPTH_MKC_MAX_SAMPLES 4096   /* most calibration sequences of one topth_calibrate_mkc call */
#define TOPTH_MKC_MAX_KEYS 32768     /* longest key range of topth_calibrate_mkc */
#define TOPTH_NOALLOC_SCRATCH_BYTES (80u << 20)   /* static scratch of topth_decode_noalloc, per GPU */

/* Human-readable text of a status code (static storage). */
const char* topth_strerror(int status);

/*
 * Bytes of device workspace an operation needs.  Arguments (unused ones are
 * ignored):
 *   TOPTH_OP_CALIBRATE: B = sequences per call S, Hq, Hkv, Lq, Lk, d, n_k
 *   TOPTH_OP_PREFILL:   B, Hq, Hkv, Lq = Lk = L, d
 *   TOPTH_OP_DECODE:    B, Hq, Hkv, Lk = Lmax, d
 *   TOPTH_OP_CALIBRATE_PRE_E: as TOPTH_OP_CALIBRATE (topth_calibrate_pre also
 *                       collecting the discarded mass; without it, the
 *                       TOPTH_OP_CALIBRATE size serves)
 *   TOPTH_OP_CALIBRATE_MKC: B = sequences S, Hq, Hkv, Lq, Lk, d (n_k ignored)
 *   TOPTH_OP_PREFILL and TOPTH_OP_DECODE sizes serve the _pre calls too.
 * Returns 0 for arguments no call could accept.
 */
size_t topth_workspace_size(int op, int B, int Hq, int Hkv, int Lq, int Lk, int d, int n_k);

/* Prepare a workspace (device, ws_bytes) on the stream: the header is zeroed
 * (status 0, default spin limit) and every exchange slot after it marked
 * empty.  Needed before the first decode call that uses it, and after a call
 * that set the status (see "Workspace"). */
int topth_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Status word of a decode workspace (0, or a combination of
 * TOPTH_STATUS_EXCHANGE_TIMEOUT), as left by the work enqueued on the stream
 * so far: the call waits for that work to finish (it synchronises the
 * stream), then copies the word to *status (host).  ws device, ws_bytes >=
 * TOPTH_WS_HEADER_BYTES. */
int topth_workspace_status(const void* ws, size_t ws_bytes, int* status, void* stream);

/* Number of polls an exchange wait of later decode calls on this workspace
 * makes before it gives up; 0 restores the default.  Enqueued on the stream
 * (no synchronisation); topth_workspace_init also restores the default.  A
 * small limit makes waits give up whenever one chunk runs ahead of another,
 * so the exchange-failure path can be exercised with every kernel still
 * ending normally.  ws device, ws_bytes >= TOPTH_WS_HEADER_BYTES. */
int topth_workspace_set_spin_limit(void* ws, size_t ws_bytes, unsigned limit, void* stream);

/*
 * Calibration, Algorithm 1 of the paper adapted to post-softmax values
 * (Sec. 3.1): for every sequence s < S, query head h, query row i (position
 * p = q_pos0 + i, seeing keys 0..p) and target k = ks[t] with p + 1 > k,
 * take the k-th largest post-softmax value of the row and add it, its square
 * and a count of one into sum/sumsq/count[t][h][p] (rows p >= n_rows are
 * skipped).  Sequences are added in order 0..S-1 for every entry, so repeated
 * calls accumulate deterministically.
 *   q      device [S][Hq][Lq][d]            k  device [S][Hkv][Lk][d]
 *   q_pos0 position of query row 0: 0 for prefill-style calibration
 *          (Lq == Lk), Lk - 1 for decode-style calibration (Lq == 1)
 *   ks     host [n_k], 1 <= ks[t] ; 1 <= n_k <= TOPTH_MAX_NK
 *   sum, sumsq device double [n_k][Hq][n_rows]; count device int same shape.
 *          The caller zeroes them before the first call of a calibration.
 *   scale  score scale, normally 1/sqrt(d)
 *   ws     device workspace, topth_workspace_size(TOPTH_OP_CALIBRATE, ...)
 */
int topth_calibrate(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk,
                    int d, int dtype, float scale, int q_pos0, const int* ks, int n_k,
                    double* sum, double* sumsq, int* count, int n_rows,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * Multi-k cumulative calibration (Appendix D, Algorithm 2 and Eq. 8): instead
 * of one threshold per target k, the S calibration samples of a row are
 * merged into kbar(theta), the mean over the samples whose value range
 * contains theta of the number of elements theta keeps, and theta(k) is read
 * back for any k.  For every query head h and query row i (position
 * p = q_pos0 + i, keys 0..p, m = p + 1 values per sample) and every target
 * ks[t]:
 *   theta[t][h][p] = max { theta : kbar(theta) >= ks[t] },
 * a sample value (the k-th largest value when S = 1), or -INFINITY (keep all)
 * where kbar never reaches ks[t] (always when ks[t] >= m).  A sample's range
 * is (its minimum, its maximum] and it keeps #{v >= theta} (the >= of every
 * compare in this library; the paper writes the count of elements greater
 * than theta).  Values are post-softmax s (pre = 0) or the scores
 * a = scale * q.k (pre = 1).  Rows p >= n_rows are not written; other rows of
 * theta are left as they are.  MKC needs every sample of a row at once, so
 * all S sequences come in one call (a long prefill can be calibrated in
 * slices of rows with q_pos0).
 *   q device [S][Hq][Lq][d], k device [S][Hkv][Lk][d]; 1 <= S <=
 *   TOPTH_MKC_MAX_SAMPLES, Lk <= TOPTH_MKC_MAX_KEYS, q_pos0 + Lq <= Lk;
 *   ks host [n_k], 1 <= n_k <= TOPTH_MKC_MAX_TARGETS, ks[t] >= 1;
 *   theta device float [n_k][Hq][n_rows];
 *   ws device, topth_workspace_size(TOPTH_OP_CALIBRATE_MKC, S, Hq, Hkv, Lq,
 *   Lk, d, 0) bytes (the pooled values twice: 8 * S * Hq * Lq * Lk bytes).
 * Results are exact for the float32 values the kernels compute (integer
 * counts over a sort), so they do not vary from launch to launch.
 */
int topth_calibrate_mkc(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk, int d,
                        int dtype, float scale, int q_pos0, int pre, const int* ks, int n_k,
                        float* theta, int n_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * Final step of Algorithm 1: theta[t][h][p] = sum/count + alpha * std
 * (population std from sumsq) for rows that were observed; -INFINITY for rows
 * with p + 1 <= ks[t]; any other row copies the nearest observed row of the
 * same (t, h) (the smaller row on a tie), or -INFINITY if none was observed.
 *   sum, sumsq, count device [n_k][Hq][n_rows]; ks host [n_k];
 *   theta device float [n_k][Hq][n_rows] (output).
 */
int topth_calibrate_finalize(const double* sum, const double* sumsq, const int* count,
                             const int* ks, int n_k, int Hq, int n_rows, float alpha,
                             float* theta, void* stream);

/*
 * Causal Top-theta prefill (Sec. 2.2 prefill phase with Sec. 3 thresholding):
 * for every (b, h, p): s = softmax over keys 0..p of scale * q.k, keep
 * s >= theta[h][min(p, n_rows-1)], out = sum_kept s_j V_j (exact SDC), plus
 * beta * mu_p with TOPTH_VMC, where beta = 1 - sum_kept s and mu_p is the mean
 * of V rows 0..p.  With TOPTH_SDC_NONE the kept weights are divided by their
 * sum (out = 0 for a row that keeps nothing) and beta = 0.
 *   q device [B][Hq][L][d]; k, v device [B][Hkv][L][d]; theta device
 *   [Hq][n_rows]; out device [B][Hq][L][d] of the input dtype (float32
 *   with TOPTH_OUT_F32);
 *   kept_count device int [B][Hq][L] or NULL; beta device float [B][Hq][L]
 *   or NULL; kept_mask device uint8 [B][Hq][L][L] or NULL: 1 where key j <= p
 *   is kept by row p (entries j > p are not written); ws device, or NULL
 *   without TOPTH_VMC.  With topth_workspace_size(TOPTH_OP_PREFILL, ...)
 *   bytes the bfloat16 path copies V to float16 there and, when every V
 *   element is within 16 in magnitude, forms P V in float16 (P scaled by 2^7
 *   and rounded to float16: under 8.1e-3 absolute error per output for
 *   L <= 65536); otherwise, or
 *   with a smaller workspace (VMC needs the first B*Hkv*L*d floats of it for
 *   the prefix means), P V uses a bfloat16 high/low split of P.
 */
int topth_prefill(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int L,
                  int d, int dtype, float scale, const float* theta, int n_rows,
                  unsigned flags, void* out, int* kept_count, float* beta,
                  unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream);

/*
 * One generative-decoding step (Sec. 2.2 decode phase, Sec. 3 thresholding):
 * for every (b, h) with n = seq_lens[b] cached keys: s = softmax over keys
 * 0..n-1 of scale * q.k, keep s >= theta[h][min(n-1, n_rows-1)], and read
 * only the V rows that some head of the GQA group keeps (Sec. 4.6).
 * out = sum_kept s_j V_j (+ beta * v_mean with TOPTH_VMC); TOPTH_SDC_NONE as
 * in topth_prefill.
 *   q device [B][Hq][d]; k_cache, v_cache device [B][Hkv][Lmax][d];
 *   seq_lens device int [B], 1 <= n <= Lmax (values outside are clamped to
 *   that range); theta device [Hq][n_rows];
 *   v_mean device float [B][Hkv][d], the running mean of the first n V rows
 *   (Sec. 3.2.2), required iff TOPTH_VMC; out device [B][Hq][d] of the input
 *   dtype (float32 with TOPTH_OUT_F32); kept_count device int [B][Hq] or NULL; beta device float [B][Hq]
 *   or NULL; vrows_read device int [B][Hkv] or NULL: number of distinct V
 *   rows read for the group (the union of its heads' kept keys);
 *   kept_mask device uint8 [B][Hq][Lmax] or NULL: 1 where key j < n is kept
 *   (entries j >= n are left untouched);
 *   ws device, zero-initialised once, topth_workspace_size(TOPTH_OP_DECODE, ...).
 */
int topth_decode(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                 int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                 const float* theta, int n_rows, const float* v_mean, unsigned flags,
                 void* out, int* kept_count, float* beta, int* vrows_read,
                 unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream);

/*
 * topth_decode for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Arguments, results, flags and errors as
 * topth_decode, without ws / ws_bytes.  The call allocates nothing: its
 * workspace is a static device array of TOPTH_NOALLOC_SCRATCH_BYTES (80 MiB)
 * inside the library, one copy on each GPU the library runs on, held until
 * the process ends.  Each call enqueues a small kernel that prepares the part
 * of the array it uses (header zero, exchange slots empty), then the decode
 * kernels, so nothing a previous call left there is read; an exchange that
 * gives up shows only as poisoned outputs of the affected groups (see
 * "Exchange failures").  Shapes whose workspace would exceed the array (the
 * exchange slots plus 4 * max(g, 4) bytes per cached key of every (batch,
 * KV head); batch 8 x 8 KV heads x 32768 keys at g = 8 needs 68 MiB) return
 * TOPTH_ESCRATCH before anything is enqueued.  All calls on one GPU share the
 * array: calls that overlap in time on that GPU (on different streams, or
 * from different host threads) race and may return wrong results.
 */
int topth_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                         int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                         const float* theta, int n_rows, const float* v_mean, unsigned flags,
                         void* out, int* kept_count, float* beta, int* vrows_read,
                         unsigned char* kept_mask, void* stream);

/*
 * Mean of the first n = seq_lens[b] V rows of each (b, kv head): the mu of
 * VMC (Sec. 3.2.2, Eq. 5) that topth_decode takes as v_mean.
 *   v device [B][Hkv][Lmax][d]; seq_lens device int [B]; v_mean device float
 *   [B][Hkv][d] (output).
 */
int topth_vmean(const void* v, const int* seq_lens, int B, int Hkv, int Lmax, int d, int dtype,
                float* v_mean, void* stream);

/*
 * One decoding step that also keeps the running V mean (Sec. 3.2.2, after
 * Eq. 7: during generation mu is maintained as a running mean).  Arguments
 * and results as topth_decode, except v_mean, which is read and written:
 *   v_mean device float [B][Hkv][d], required.  On entry it holds the mean of
 *          V rows 0..n-2 of each (b, kv head), n = seq_lens[b] clamped to
 *          [1, Lmax] (ignored when n = 1); row n-1 is the token just appended.
 *          On return it holds the mean of rows 0..n-1, ((n-1) mu + V[n-1]) / n
 *          formed in float64 and stored as float, and that is the mu the VMC
 *          term of this step uses.  It is updated whatever the flags are.
 * The result equals topth_vmean_append(old = n-1, new = n) followed by
 * topth_decode.  For bf16 the update runs inside the decode kernel (no extra
 * launch); for fp32 the update kernel runs first on the same stream.  Calling
 * twice for the same n appends row n-1 twice.  Errors as topth_decode;
 * TOPTH_EINVAL also for v_mean == NULL.
 */
int topth_decode_append(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                        int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                        const float* theta, int n_rows, float* v_mean, unsigned flags,
                        void* out, int* kept_count, float* beta, int* vrows_read,
                        unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Pre-softmax Top-theta (the paper's Algorithm 1 in its printed form, and
 * Sec. 3.2.1): thresholds are on the scores a = scale * q.k themselves, in
 * score units, and the kept elements are weighted by softmax over the kept
 * scores times R / (R + E~) (Eq. 4), where R and E are the sums of exp(a - max a)
 * over the kept and the discarded elements and E~ estimates E.  VMC adds
 * beta * mu with beta = E~ / (R + E~) (Sec. 3.2.2, case (ii)).
 * ------------------------------------------------------------------------ */

/*
 * Calibration in the pre-softmax form: as topth_calibrate, but the sample of
 * a row is its k-th largest score a (not a post-softmax value).  With
 * esum != NULL the call also adds, per row, the discarded mass of the row's
 * top-k selection, E = sum over the elements outside the k largest of
 * exp(a - max a), into esum[t][h][p] (device double, same shape as sum; the
 * offline estimate of E~, Sec. 3.2.1 item 1).  ws must then hold
 * topth_workspace_size(TOPTH_OP_CALIBRATE_PRE_E, ...) bytes.  The thresholds
 * come from topth_calibrate_finalize, the E~ table from
 * topth_calibrate_finalize_etilde.
 */
int topth_calibrate_pre(const void* q, const void* k, int S, int Hq, int Hkv, int Lq, int Lk,
                        int d, int dtype, float scale, int q_pos0, const int* ks, int n_k,
                        double* sum, double* sumsq, int* count, double* esum, int n_rows,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Offline E~ table from the sums of topth_calibrate_pre: e_tilde[t][h][p] =
 * esum / count for observed rows; 0 for rows with p + 1 <= ks[t] (nothing is
 * discarded); any other row copies the nearest observed row of the same (t, h)
 * (the smaller row on a tie), or 0 if none was observed.
 *   esum device double, count device int [n_k][Hq][n_rows]; ks host [n_k];
 *   e_tilde device float [n_k][Hq][n_rows] (output).
 */
int topth_calibrate_finalize_etilde(const double* esum, const int* count, const int* ks, int n_k,
                                    int Hq, int n_rows, float* e_tilde, void* stream);

/*
 * Causal pre-softmax prefill: keep a >= theta[h][min(p, n_rows-1)] (theta in
 * score units, -INFINITY keeps all); out = sum_kept w_j V_j (+ beta * mu_p
 * with TOPTH_VMC), w_j = exp(a_j - max a) / (R + E~), with E~ by flags:
 * exact E (default), TOPTH_SDC_EXPTH (gamma >= 0), TOPTH_SDC_OFFLINE (e_tilde
 * device float [Hq][n_rows], required), TOPTH_SDC_NONE (E~ = 0, beta = 0).  A
 * row with R + E~ = 0 outputs 0 with beta = 0.  At most one of the three
 * estimate flags.  Other arguments as topth_prefill; the bfloat16 path makes
 * one sweep over the keys (no row log-sum-exp pass).
 */
int topth_prefill_pre(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int L,
                      int d, int dtype, float scale, const float* theta, const float* e_tilde,
                      int n_rows, unsigned flags, float gamma, void* out, int* kept_count,
                      float* beta, unsigned char* kept_mask, void* ws, size_t ws_bytes, void* stream);

/*
 * One pre-softmax decoding step: keep a >= theta[h][min(n-1, n_rows-1)] and
 * weight as topth_prefill_pre (n = seq_lens[b] keys); v_mean is required iff
 * TOPTH_VMC without TOPTH_SDC_NONE.  Other arguments, the workspace contract
 * and vrows_read as topth_decode.
 */
int topth_decode_pre(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                     int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                     const float* theta, const float* e_tilde, int n_rows, const float* v_mean,
                     unsigned flags, float gamma, void* out, int* kept_count, float* beta,
                     int* vrows_read, unsigned char* kept_mask, void* ws, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Decode-serving helpers
 * ------------------------------------------------------------------------ */

/*
 * Running mean of V for VMC (Sec. 3.2.2: during generative decoding mu is kept
 * as a running mean instead of being recomputed): after rows
 * old_lens[b] .. new_lens[b]-1 of each (b, KV head) have been written to the
 * cache, v_mean (the mean of the first old_lens[b] rows on entry) becomes the
 * mean of the first new_lens[b] rows: (old * mu + sum of the new rows) / new.
 * A batch element with old_lens[b] = 0 starts fresh (v_mean is not read).
 *   v_cache device [B][Hkv][Lmax][d]; old_lens, new_lens device int [B]
 *   (clamped to 1 <= new <= Lmax and 0 <= old <= new); v_mean device float
 *   [B][Hkv][d], updated in place.  The sums are float64 in row order.
 */
int topth_vmean_append(const void* v_cache, const int* old_lens, const int* new_lens, int B, int Hkv,
                       int Lmax, int d, int dtype, float* v_mean, void* stream);

/*
 * Thresholds as a function of the row position, for rows no calibration
 * sequence reached (the paper fits the per-row thresholds to the sequence
 * length; the function is not given, so this library uses a least-squares
 * polynomial of degree 0..3 in x = ln(p + 1)).  topth_theta_fit fits, per
 * (t, h), the rows with count > 0 and p + 1 >= min_len_over_k * ks[t] of a
 * finalized slab: on ln(theta) when log_domain != 0 (post-softmax thresholds,
 * which fall roughly as a power of the row length; rows with theta <= 0 are
 * skipped), on theta otherwise (pre-softmax thresholds).  Rows just above
 * p + 1 = k do not follow that trend (the k-th largest value sits near the
 * row's minimum there, so thresholds first rise with the row length): fits
 * that include them and are extrapolated to much longer rows keep far too
 * few or far too many keys.  min_len_over_k = 4 leaves them out and is the
 * recommended setting; 0 fits every observed row.
 *   ks host [n_k], the target k of each slab; min_len_over_k >= 0;
 *   theta device float, count device int [n_k][Hq][n_rows];
 *   coef device double [n_k][Hq][degree + 1], highest power first (output);
 *   NaN coefficients where fewer than degree + 1 rows are usable.  The fit
 *   solves the normal equations in float64: a cubic over a narrow range of
 *   ln(p + 1) is ill-conditioned, and its coefficients (not its values) may
 *   then differ in the leading digits from an orthogonal-factorisation solve.
 */
int topth_theta_fit(const float* theta, const int* count, const int* ks, int n_k, int Hq, int n_rows,
                    int degree, int log_domain, int min_len_over_k, double* coef, void* stream);

/*
 * Evaluate fitted thresholds into a slab of n_out rows (which may be longer
 * than the calibrated one): theta_out[t][h][p] = poly(ln(p + 1)), exponentiated
 * when log_domain != 0, for p + 1 > ks[t]; -INFINITY (keep all) below.
 *   coef device double [n_k][Hq][degree + 1]; ks host [n_k];
 *   theta_out device float [n_k][Hq][n_out] (output).
 */
int topth_theta_eval(const double* coef, const int* ks, int n_k, int Hq, int degree, int log_domain,
                     int n_out, float* theta_out, void* stream);

/*
 * One decoding step with the GQA selection variants of Sec. 4.6 (post-softmax
 * thresholds, as topth_decode): a key is loaded for a (batch, KV head) group
 * when at least min_votes (1 .. Hq/Hkv) of the group's heads keep it
 * (s >= theta), which discards V rows requested by only a few heads; with
 * augment = 0 each head then uses its own kept keys among the loaded ones,
 * with augment = 1 every head uses all loaded keys (each head's selection
 * widened to the whole group's), weighted by its own post-softmax values.  min_votes = 1, augment = 0 is topth_decode.  kept_count counts the
 * keys a head uses; vrows_read the loaded keys; kept_mask marks, per head, the
 * keys it uses.  Other arguments and the workspace contract as topth_decode.
 */
int topth_decode_gqa(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                     int B, int Hq, int Hkv, int Lmax, int d, int dtype, float scale,
                     const float* theta, int n_rows, const float* v_mean, unsigned flags,
                     int min_votes, int augment, void* out, int* kept_count, float* beta,
                     int* vrows_read, unsigned char* kept_mask, void* ws, size_t ws_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOPTH_H */
