/*
 * sekv.h -- C ABI of the SeKV decode path on MI355X (gfx950).
 *
 * The method is the hierarchical, resolution-adaptive KV cache of the SeKV
 * article (aitrends.kr/articles/75020).  Section names below refer to it:
 *   [Contrib] 핵심 기여 (Key contributions)   [Method] 방법론 (Method, Fig. 2)
 *   [Tech]    기술 상세 (Technical details)
 *
 * Prefill builds an index (sekv_build_index): surprisal span split, per-span
 * surprisal-weighted mean K/V and d'-dim summary keys in HBM, truncated-SVD
 * factors per (layer, KV head, span) in HBM or in pinned host memory.  Each
 * decode step routes (sekv_route) and attends (sekv_decode_attend).
 *
 * Conventions (every call):
 *  - Returns a sekv_status.  On any status other than SEKV_OK no output has
 *    been written and the index is unchanged; sekv_last_error() returns a
 *    message for the calling thread's last failure.  Arguments are checked on
 *    the host before any HIP call.
 *  - "device" pointers are HIP device memory on the context's device; "host"
 *    pointers are ordinary host memory.  The caller owns every buffer it
 *    passes and the library never frees or retains them past the call, except
 *    where a call says it copies them.  The library owns sekv_ctx, sekv_index,
 *    the pinned host factor pool and the HBM staging ring.
 *  - Device work is enqueued on the context's HIP stream and is asynchronous:
 *    device outputs are valid once the caller synchronises that stream.
 *    Calls that must read device data on the host (build, import/export, the
 *    pinned-tier gather) synchronise the stream internally and say so.
 *  - Layouts are row-major, bf16 is IEEE bfloat16 stored in uint16_t, fp32
 *    is float.  Indices: b batch, l layer, h query head, g = h / G KV head,
 *    G = Hq / Hkv, S span ordinal (position order), d head dim, d' = dprime.
 *  - One context per host thread.  An index may be used by many decode calls
 *    on the context that built it; calls on one stream are ordered.
 */
#ifndef SEKV_H
#define SEKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SEKV_OK = 0,
  SEKV_EINVAL = 1,       /* bad argument (null, shape, range)                 */
  SEKV_ENOMEM = 2,       /* device or pinned host allocation failed           */
  SEKV_EHIP = 3,         /* a HIP runtime call failed (message has the text)  */
  SEKV_ECAPACITY = 4,    /* a fixed-size buffer too small for this call: the
                            staging ring for its union, or the no-allocation
                            decode's scratch                                  */
  SEKV_ESTATE = 5,       /* object used after free or on the wrong context    */
  SEKV_EUNSUPPORTED = 6  /* shape not compiled (d, G or R outside the set)    */
} sekv_status;

typedef enum {
  SEKV_TIER_HBM = 0,          /* span factors resident in HBM                   */
  SEKV_TIER_PINNED_HOST = 1   /* span factors in pinned host memory; each decode
                                 call gathers the routed spans into an HBM ring */
} sekv_tier;

typedef struct sekv_ctx sekv_ctx;
typedef struct sekv_index sekv_index;

/* Shapes and prefill settings.  Supported: d in {64, 128}; G in {1, 2, 4, 8};
 * R in {16, 32, 64} with R <= d; 1 <= dprime <= 64; l_min >= 1. */
typedef struct {
  int32_t B, L, Hq, Hkv, d, T;
  int32_t R;            /* max SVD rank per span                                  */
  int32_t dprime;       /* summary-key dimension d'                              */
  float alpha_sp;       /* span boundary where H_t > mu + alpha_sp * sigma       */
  int32_t l_min;        /* anchor-free runs shorter than l_min stay raw          */
  int32_t oversample;   /* randomized-SVD oversampling p (sketch width R + p)    */
  int32_t power_iters;  /* randomized-SVD power iterations q                     */
  uint64_t seed;        /* Gaussian test matrices: Philox4x32-10 keyed by seed   */
  int32_t tier;         /* sekv_tier                                             */
  int64_t ring_bytes;   /* pinned tier: HBM staging ring size, 0 = two slots of
                           the largest layer's whole factor set.  Each slot
                           mirrors one layer's region of the pool; one slot is
                           required (ECAPACITY otherwise), and with two a call
                           over several layers gathers the next layer while the
                           current one is attended                               */
  float gate_eps;       /* variable effective rank ([Contrib], dual resolution;
                           [Tech], low-rank paragraph: the gates set each span's
                           effective rank and components are dropped at storage
                           and transfer): when > 0, component i of a span's K
                           (V) factorization is stored only if its gate
                           m_i >= gate_eps.  <= 0 keeps every component.  Each
                           blob keeps min(R, n_S) components at most, padded
                           with zero components to a multiple of 16 (>= 16).
                           NaN is rejected (EINVAL).                             */
} sekv_build_params;

/* Index summary. */
typedef struct {
  int32_t B, L, Hq, Hkv, d, R, dprime, tier;
  int32_t max_spans;         /* max over b of N_S(b)                             */
  int32_t mask_words;        /* ceil(max_spans / 64): words per (b, l, h) mask   */
  int64_t total_spans;       /* sum over b of N_S(b)                             */
  int64_t total_raw;         /* sum over b of N_raw(b)                           */
  int64_t total_span_tokens; /* sum over b, S of n_S                             */
  int64_t resident_bytes;    /* HBM: K/V rows (raw + pseudo), s, W copy          */
  int64_t factor_bytes;      /* factor pool (HBM or pinned host)                 */
  int64_t ring_bytes;        /* HBM staging ring (pinned tier), else 0           */
} sekv_index_info;

/* Host-side logical layout of an index, used by import and export.  Every
 * array is concatenated over b in order; per b the shapes are:
 *   span_start, span_len   int32 [N_S(b)]        spans in position order
 *   raw_pos                int32 [N_raw(b)]      raw token positions, ascending
 *   k_res, v_res           bf16  [L][Hkv][N_raw(b) + N_S(b)][d]
 *                          rows: raw tokens (raw_pos order), then one pseudo
 *                          row per span (the surprisal-weighted mean)
 *   s                      fp32  [L][Hq][d'][N_S(b)]  summary keys
 *   uk, uv                 bf16  [L][Hkv][sum_S n_S][R]  left factors, span S
 *                          at row offset sum_{S'<S} n_S'
 *   vkt, vvt               bf16  [L][Hkv][N_S(b)][R][d]  right factors (V^T)
 *   smk, smv               fp32  [L][Hkv][N_S(b)][R]     sigma_i * m_i
 * plus W, fp32 [L][Hq][d'][d], the routing projection (not per b).
 * Import reads these (host, const); export writes them into caller buffers
 * sized from sekv_index_info / sekv_index_counts.  The stored rank of each
 * imported K (V) factorization is the number of components up to its last
 * nonzero sigma_i * m_i, rounded up to 16: trailing zero components are
 * not stored (they contribute nothing). */
typedef struct {
  const int32_t* n_spans;     /* [B] */
  const int32_t* n_raw;       /* [B] */
  const int32_t* span_start;
  const int32_t* span_len;
  const int32_t* raw_pos;
  const uint16_t* k_res;
  const uint16_t* v_res;
  const float* s;
  const uint16_t* uk;
  const uint16_t* uv;
  const uint16_t* vkt;
  const uint16_t* vvt;
  const float* smk;
  const float* smv;
  const float* W;
} sekv_host_index;

typedef struct {
  int32_t* span_start;
  int32_t* span_len;
  int32_t* raw_pos;
  uint16_t* k_res;
  uint16_t* v_res;
  float* s;
  uint16_t* uk;
  uint16_t* uv;
  uint16_t* vkt;
  uint16_t* vvt;
  float* smk;
  float* smv;
  int32_t* rank;        /* [L][Hkv][N_S(b)][2]: stored components (K, V) of each
                           blob, multiples of 16; components past them export
                           as zeros.  Nullable, like every member.               */
} sekv_host_index_out;

/* Per-call decode statistics.  The gather fields are filled for the pinned
 * tier only (zero for the HBM tier). */
typedef struct {
  uint64_t union_spans;    /* sum over (b, l, g) of |union of the G heads' z|   */
  uint64_t pcie_bytes;     /* bytes moved host -> HBM ring (padded blobs)        */
  uint64_t pcie_copies;    /* gather kernel launches (one per layer)             */
  double pcie_ms;          /* summed stream time of the gather launches (HIP
                              events around each); overlapped with attention
                              when the call gathers one layer ahead             */
} sekv_stats;

/* ---------------------------------------------------------------- lifecycle */

/* Create a context on HIP device `device`.  `stream` is a hipStream_t to
 * enqueue on (borrowed, must outlive the context) or NULL for the legacy
 * default stream.  *out receives the context. */
sekv_status sekv_create(int32_t device, void* stream, sekv_ctx** out);

/* Destroy a context (waits for its stream).  NULL is a no-op. */
void sekv_destroy(sekv_ctx* ctx);

/* Message of the calling thread's last failing call ("" if none). */
const char* sekv_last_error(void);

/* Upper bound on the number of compressed spans of a T-token context:
 * k spans of >= l_min tokens need k*l_min tokens plus k-1 separating
 * anchors, so k <= (T + 1) / (l_min + 1).  Sizes the gate array. */
int32_t sekv_max_spans(int32_t T, int32_t l_min);

/* Host-only check of build/import parameters, the same check the build and
 * import calls run before any HIP call (no device needed). */
sekv_status sekv_validate_params(const sekv_build_params* p);

/* ------------------------------------------------------------------ prefill */

/* Build the index of B sequences ([Method]: span split at H_t > mu +
 * alpha*sigma with the boundary tokens kept as anchors; per span a
 * surprisal-weighted mean key/value and a d'-dim summary key s = W k̄ on the
 * GPU; a truncated SVD U Sigma V^T of the span's keys and values per layer
 * and KV head, computed by randomized subspace iteration ([Method]: the
 * randomized truncated SVD that parallelises prefill; [Tech]).  Anchors and
 * runs shorter than l_min stay raw ([Method]).
 *   K, V   device bf16 [B][L][Hkv][T][d], 16-byte aligned
 *   H      device fp32 [B][T]  token surprisal (>= 0, finite)
 *   W      device fp32 [L][Hq][d'][d]  routing projection (copied into the
 *          index), 16-byte aligned
 *   (a misaligned K, V or W is SEKV_EINVAL, refused before any work)
 *   gates  device fp32 [B][L][Hkv][2 (K|V)][S_max][R] component gates m, span
 *          ordinal S using slot S, S_max = sekv_max_spans(T, l_min); or NULL
 *          for m = 1.  sigma*m is stored.
 * Synchronises the stream (span counts decide the index size). */
sekv_status sekv_build_index(sekv_ctx* ctx, const sekv_build_params* p,
                             const void* K, const void* V, const float* H,
                             const float* W, const float* gates, sekv_index** out);

/* The randomized truncated SVD the index build runs on every span matrix
 * ([Method]: randomized truncated SVD of each span's key and value matrix;
 * Halko-Martinsson-Tropp subspace iteration with sketch width R + oversample,
 * power_iters power steps, Gaussian test matrix from Philox4x32-10 keyed by
 * seed and matrix index), exposed on a batch of arbitrary matrices with fp32
 * outputs, before the bf16 storage rounding of the index.
 *   A        device bf16, matrix m is rows [row_off[m], row_off[m] + rows[m])
 *            of a row-major [*][d] array
 *   row_off  device int64 [count];  rows  device int32 [count], each >= 1
 *   U        device fp32 [count][max_rows][R]   left factors (rows >= rows[m]
 *            and columns past the numerical rank are zero)
 *   sigma    device fp32 [count][R]  non-increasing, >= 0
 *   Vt       device fp32 [count][R][d]  right factors (rows)
 * d in {64, 128}, R in [1, 64], R <= d, max_rows >= every rows[m] (not
 * checked on the device: the caller guarantees it). */
sekv_status sekv_rsvd_batched(sekv_ctx* ctx, int32_t count, const void* A, const int64_t* row_off,
                              const int32_t* rows, int32_t max_rows, int32_t d, int32_t R,
                              int32_t oversample, int32_t power_iters, uint64_t seed,
                              float* U, float* sigma, float* Vt);

/* Build an index from host arrays in the logical layout above (tests,
 * resume).  p->B, L, Hq, Hkv, d, R, dprime, tier, ring_bytes are used; the
 * span tables must partition [0, T) with spans of length >= 1.  Copies the
 * data; synchronises the stream. */
sekv_status sekv_index_import(sekv_ctx* ctx, const sekv_build_params* p,
                              const sekv_host_index* h, sekv_index** out);

/* Copy an index back into caller host buffers (logical layout above).  Any
 * NULL member of `h` is skipped.  Synchronises the stream. */
sekv_status sekv_index_export(sekv_ctx* ctx, const sekv_index* idx,
                              const sekv_host_index_out* h);

/* As sekv_index_export for sequences [seq_begin, seq_begin + seq_count) and
 * layers [layer_begin, layer_begin + layer_count) only: the logical layout
 * of those sequences (concatenated in order), with layer_count in place of L
 * (layer layer_begin first).  SEKV_EINVAL for a range outside [0, B) or
 * [0, L).  Synchronises the stream. */
sekv_status sekv_index_export_part(sekv_ctx* ctx, const sekv_index* idx, int32_t seq_begin,
                                   int32_t seq_count, int32_t layer_begin, int32_t layer_count,
                                   const sekv_host_index_out* h);

sekv_status sekv_index_get_info(const sekv_index* idx, sekv_index_info* info);

/* Per-sequence counts: n_spans[b] = N_S(b), n_raw[b] = N_raw(b) (host [B]). */
sekv_status sekv_index_counts(const sekv_index* idx, int32_t* n_spans, int32_t* n_raw);

/* Free an index (waits for the context stream).  NULL is a no-op. */
void sekv_index_free(sekv_index* idx);

/* ------------------------------------------------------------------- decode */

/* Stage 1 routing ([Method]; [Tech]) for layers [layer_begin, layer_begin +
 * layer_count): u = W^(l,h) q^(l,h); score a_S = u . s_S (fp32);
 * alpha_S = sigmoid(a_S); z_S = [alpha_S > tau^(l,h)].  The sigmoid is
 * strictly increasing, so z_S is decided as a_S > logit(tau) = ln(tau / (1 -
 * tau)), taken in fp64 from the fp32 tau (every span for tau <= 0, none for
 * tau >= 1 or NaN): the same decision in exact arithmetic, and exact where
 * alpha rounds to 1 in fp32.  With cap > 0, a (b, l, h) with more than cap
 * expansions keeps the cap largest a_S (the order of alpha), ties to the
 * lower span index ([Tech]: spans taken in descending alpha until the budget
 * holds).
 *   q      device bf16 [B][layer_count][Hq][d], 16-byte aligned
 *   tau    device fp32 [layer_count][Hq]  (+-inf allowed)
 *   mask   device uint64 [B][layer_count][Hq][mask_words], 8-byte aligned;
 *          bit j of word w is z of span 64w + j; bits at or past N_S(b) are 0
 *   (a misaligned q or mask is SEKV_EINVAL, refused before any work)
 *   alpha  device fp32 [B][layer_count][Hq][mask_words * 64], 16-byte
 *          aligned (SEKV_EINVAL otherwise), or NULL: sigmoid(a_S) in fp32,
 *          for inspection; entries at or past N_S(b) are unspecified
 * With cap > 0 the call uses index-owned scratch for the scores (grown on
 * first use); calls on one context are ordered on its stream. */
sekv_status sekv_route(sekv_ctx* ctx, const sekv_index* idx, int32_t layer_begin,
                       int32_t layer_count, const void* q, const float* tau,
                       int32_t cap, uint64_t* mask, float* alpha);

/* Stage 1 routing as sekv_route with no per-head cap, then the budget rule
 * ([Tech]: spans taken in descending alpha until the budget holds) applied to
 * a pool: for each sequence b, over every (layer, head, span) triple of the
 * call, keep the budget largest scores a_S (the order of alpha) among the
 * routed triples, ties to the lower (layer, head, span) position (the flat
 * order of the mask words).
 * A call over one layer pools that layer's heads; a call over all layers
 * pools the whole model (which needs every layer's query at once: a decode
 * loop whose layer l + 1 query depends on layer l pools per layer).
 * budget 0 = no budget; budget < 0 is SEKV_EINVAL.
 *   q, tau, mask, alpha  as for sekv_route
 * With budget > 0 the call uses index-owned score scratch, as sekv_route with
 * a cap does. */
sekv_status sekv_route_pooled(sekv_ctx* ctx, const sekv_index* idx, int32_t layer_begin,
                              int32_t layer_count, const void* q, const float* tau,
                              int32_t budget, uint64_t* mask, float* alpha);

/* Place tau per (l, h) from a calibration query so that k = round(frac * sum_b
 * N_S(b)) of the (b, span) pairs exceed it: the midpoint of the k-th and
 * (k+1)-th largest alpha, k clipped to [1, sum_b N_S(b) - 1].  The pages learn
 * tau; this stands in for the learned value on synthetic workloads.
 *   q_cal  device bf16 [B][layer_count][Hq][d], 16-byte aligned (SEKV_EINVAL
 *          otherwise);  tau_out device fp32 [layer_count][Hq] */
sekv_status sekv_calibrate_tau(sekv_ctx* ctx, const sekv_index* idx, int32_t layer_begin,
                               int32_t layer_count, const void* q_cal, float frac,
                               float* tau_out);

/* Stage 2 and attention ([Method], Fig. 2; [Tech] reconstruction sum): for each
 * (b, l, h) attend over every raw row, over the pseudo row (mean key/value,
 * logit bias ln n_S) of each span with z = 0, and over the reconstructed rows
 * Khat = U^K diag(sigma m) V^K^T, Vhat likewise, of each span with z = 1.  The
 * reconstruction is evaluated in factored form and never materialised.
 * Softmax scale 1/sqrt(d).
 *   q      device bf16 [B][layer_count][Hq][d], 16-byte aligned
 *   mask   device uint64 [B][layer_count][Hq][mask_words], 8-byte aligned
 *          (from sekv_route or the caller); a misaligned q or mask is
 *          SEKV_EINVAL, refused before any work
 *   out    device fp32 [B][layer_count][Hq][d]
 *   stats  host, or NULL
 * Work: the attention kernel's workgroups each take a slice of the resident
 * rows and an equal share of the union of the G heads' routed spans of their
 * (b, l, KV head); a merge kernel combines their softmax partials.
 * Pinned tier: the routed union's factor blobs are first gathered from the
 * mapped pinned pool into the HBM staging ring by a kernel reading them over
 * PCIe ([Method] Stage 2: the factors are fetched from the CPU
 * asynchronously).  Each ring slot mirrors one layer's pool region (a blob
 * sits at its own offset), so nothing is placed on the host; the ring must
 * hold one slot (SEKV_ECAPACITY otherwise, before any device work).  With two
 * slots and layer_count > 1 the gathers run on the index's own stream one
 * layer ahead of the attention ([Method] Fig. 2: asynchronous transfer
 * overlapped with the decode pipeline), ordered by events against the call's
 * stream: the call's results are still complete when its stream is.  The
 * call does not synchronise, except when stats is non-NULL on the pinned
 * tier (to read back the union sizes and the gather times).  The index owns
 * the partials buffer (grown on first use): calls on one context are ordered
 * on its stream. */
sekv_status sekv_decode_attend(sekv_ctx* ctx, const sekv_index* idx, int32_t layer_begin,
                               int32_t layer_count, const void* q, const uint64_t* mask,
                               float* out, sekv_stats* stats);

/* sekv_decode_attend for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and arguments, with the attention items' softmax partials
 * in a static device scratch array that the library holds for each GPU until
 * the process ends (its address is taken once per device in sekv_create), so
 * the call itself calls no hipMalloc, hipFree or other allocating routine.
 * Limits and conditions:
 *  - the partials of one call, 4 * layer_count * items * G * (d + 2) bytes,
 *    must fit the 40 MiB scratch, else SEKV_ECAPACITY with nothing written
 *    (a 32-query-head, 8-KV-head 128K layer needs 1.6 MB per layer);
 *  - HBM tier only (SEKV_EUNSUPPORTED for the pinned tier, whose gather
 *    allocates its bookkeeping);
 *  - every call on one GPU shares that GPU's scratch: calls that overlap in
 *    time on one GPU (other streams or contexts) race and must be ordered by
 *    the caller;
 *  - the attention kernel is not timed (sekv_timing_enable does not apply);
 *    stats is zero-filled or NULL. */
sekv_status sekv_decode_attend_noalloc(sekv_ctx* ctx, const sekv_index* idx, int32_t layer_begin,
                                       int32_t layer_count, const void* q, const uint64_t* mask,
                                       float* out, sekv_stats* stats);

/* --------------------------------------------------------- instrumentation */

/* Kernel timing.  While enabled, every sekv_route call brackets its routing
 * kernels with HIP events on the context stream, and every sekv_decode_attend
 * call times its attention kernel (not the partial merge) with HIP events that
 * the launch itself records in its dispatch packet (hipExtLaunchKernel), so
 * their interval is the kernel's execution without the dispatch gap; nothing
 * is synchronised.  sekv_timing_read synchronises those events, returns the summed
 * milliseconds and launch counts since the previous read (or since enabling),
 * and starts a new period.  Any output pointer may be NULL. */
sekv_status sekv_timing_enable(sekv_ctx* ctx, int32_t enable);
sekv_status sekv_timing_read(sekv_ctx* ctx, double* route_ms, int64_t* route_launches,
                             double* attend_ms, int64_t* attend_launches);

#ifdef __cplusplus
}
#endif

#endif /* SEKV_H */
