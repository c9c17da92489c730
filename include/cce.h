/*
 * cce.h -- C ABI of the MI355X (gfx950) Cut Cross-Entropy library, libcce.so.
 *
 * The operation (sources, by page title and section):
 *   - "Cut Your Losses in Large-Vocabulary Language Models" (paper digest),
 *     section "The Mathematical Decomposition": per token, the log-likelihood is
 *     the target logit minus the log-sum-exp of all logits; the loss here is
 *     its negative, loss_n = lse_n - C[x_n] . E_n.
 *   - same page, Algorithm 2 (linear-log-sum-exp forward): lse over vocabulary
 *     blocks merged by log-add-exp, never storing the N x |V| logits.
 *   - same page, Algorithms 3 and 4 (backward) and "Gradient Filtering": the
 *     logits are recomputed, G = softmax - onehot(x) (the gradient of the
 *     loss; the digest prints the opposite sign, the gradient of the
 *     log-likelihood), and dE = G C, dC = G^T E, each row of G scaled by the
 *     upstream gradient; blocks whose every |G| is below eps are skipped.
 *   - kernel card "cut-cross-entropy", sections "Usage", "Correctness" and
 *     "Requirements and limits": E [N,D] and C [V,D] bf16, int64 targets,
 *     ignore_index rows contribute nothing and get exactly zero gradient, a
 *     fully masked batch gives zero loss, reductions none / mean / sum.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers into memory the caller owns,
 *     row-major and contiguous, 16-byte aligned.  E is [N, D] bf16, C is
 *     [V, D] bf16, x is [N] int64.  N >= 0, V >= 1, D >= 8 with D % 8 == 0.
 *   - `stream` is a hipStream_t (cast to void*); 0 means the null stream.
 *     Work is enqueued on it; no entry point synchronises, allocates or frees.
 *   - `workspace` is caller-owned device memory of at least the size
 *     cce_workspace_bytes reports for the same (N, V, D); its contents on
 *     entry do not matter and are clobbered.  The workspace never grows with
 *     N*V: it is O(N*D) for the forward and O(Nb*min(V, Vc) + N*D +
 *     D*min(V, Vc) + V) for the backward, where the backward's vocabulary chunk
 *     Vc is 16384 when N <= 4096 and ceil(N/256) * ceil(D/256) >= 128, else
 *     8192, and its token block Nb is N up to 16384 rows (padded to 256), past
 *     that equal blocks of whole 256-row tiles of at most 8192 rows.
 *   - Ignored rows (x[n] == ignore_index) are removed before any tile is
 *     computed ("Cut Your Losses" digest, Table A1: dropping ignored tokens
 *     ahead of the loss): both calls move the valid rows, in order, to the
 *     front of a compacted copy of E inside the workspace, run every tile on
 *     those rows only, and write the results back to the callers' rows.
 *   - Arguments are validated on the host before any launch; on error nothing
 *     is enqueued and no output is written.  A failed launch returns
 *     CCE_ERR_HIP.  Targets outside [0, V) that are not ignore_index are never
 *     used as an index: the forward gives that row a NaN loss (so a mean or
 *     sum is NaN too), the backward treats the row as ignored.
 *   - Calls that share a workspace must not overlap; otherwise entry points
 *     are reentrant and keep no state between calls (profiling aside).
 */
#ifndef CCE_H
#define CCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCE_OK = 0,
  CCE_ERR_NULL_POINTER = 1,
  CCE_ERR_BAD_SHAPE = 2,
  CCE_ERR_BAD_REDUCTION = 3,
  CCE_ERR_BAD_ALIGNMENT = 4,
  CCE_ERR_BAD_EPS = 5,
  CCE_ERR_WORKSPACE_TOO_SMALL = 6,
  CCE_ERR_HIP = 7,
  CCE_ERR_BAD_FILTER_MODE = 8,
  CCE_ERR_SCRATCH_TOO_SMALL = 9
} cce_status;

typedef enum {
  CCE_REDUCTION_NONE = 0, /* loss is [N]: per-token loss, 0 on ignored rows */
  CCE_REDUCTION_MEAN = 1, /* loss is [1]: sum over valid rows / max(N_valid, 1) */
  CCE_REDUCTION_SUM = 2   /* loss is [1]: sum over valid rows */
} cce_reduction;

/* Which contractions of the backward take the filtered G ("Cut Your Losses"
 * digest, "Numerical Stability Variants").  The digest's FullC variant leaves
 * dC unfiltered so that vocabulary rows whose probability stays below eps
 * still get a gradient (its recommendation for pretraining), FullE leaves dE
 * unfiltered.  The Kahan summation those variants pair with it answers bf16
 * accumulation; here both contractions accumulate in fp32, so it has no
 * counterpart. */
typedef enum {
  CCE_FILTER_BOTH = 0,   /* dE and dC filtered (basic CCE) */
  CCE_FILTER_FULL_C = 1, /* dE filtered, dC from the unfiltered G */
  CCE_FILTER_FULL_E = 2  /* dC filtered, dE from the unfiltered G */
} cce_filter_mode;

/* Filter statistics written by cce_backward (device memory).  A unit is
 * unit_rows consecutive valid tokens (ignored rows removed, see above) x
 * unit_cols vocabulary entries, aligned at 0 and clipped to N_valid and V;
 * units_total = ceil(N_valid/unit_rows) * ceil(V/unit_cols). */
typedef struct {
  int64_t units_total;
  int64_t units_skipped;
  int32_t unit_rows;
  int32_t unit_cols;
} cce_filter_stats;

/* Workspace sizes in bytes for cce_forward and cce_backward at (N, V, D) on
 * the current device (the launch plan fills whole rounds of its compute
 * units: 256 on an MI355X, assumed when no device can be queried).  Either
 * output pointer may be NULL. */
cce_status cce_workspace_bytes(int64_t N, int64_t V, int64_t D,
                               size_t *fwd_bytes, size_t *bwd_bytes);

/* Forward ("Cut Your Losses" digest, Algorithms 1 and 2; kernel card,
 * "Method").  Computes lse[n] = log sum_v exp(C[v].E[n]) and
 * loss_n = lse[n] - C[x[n]].E[n] in fp32 from bf16 inputs, without storing
 * the logits.  Ignored rows (x[n] == ignore_index): lse[n] = 0, loss_n = 0.
 *   loss: [N] floats for CCE_REDUCTION_NONE, [1] float otherwise (N_valid = 0
 *         gives 0).
 *   lse:  [N] floats, kept by the caller for cce_backward.
 * Results are bitwise reproducible run to run. */
cce_status cce_forward(const void *E, const void *C, const int64_t *x,
                       int64_t N, int64_t V, int64_t D, int64_t ignore_index,
                       int reduction, float *loss, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Backward ("Cut Your Losses" digest, Algorithms 3 and 4, "Gradient
 * Filtering"; CCE blog post, "Gradient filtering").  Recomputes the logits,
 * forms G = exp(A - lse) - onehot(x), zeroes every filter unit (32 valid
 * tokens x 32 vocabulary entries) whose every |G| < filter_eps (the test is
 * on the unscaled G), scales row n by s_n (grad_loss[0] / max(N_valid,1) for mean,
 * grad_loss[0] for sum, grad_loss[n] for none; 0 on ignored rows) and writes
 *   dE [N, D] bf16 = s G C    and    dC [V, D] bf16 = (s G)^T E,
 * both overwritten (beta = 0).  The contractions take s G in fp16 with a
 * power-of-two scale (11 significant bits, every |G| >= 2e-9 a normal
 * number) and E, C exactly converted to power-of-two-scaled fp16; they
 * accumulate in fp32 and round once to bf16.  Ignored rows get dE rows that
 * are exactly zero.
 *   lse:        [N] from cce_forward.
 *   grad_loss:  device, [1] for mean/sum, [N] for none.
 *   filter_eps: finite and >= 0; 0 disables the filter; 2^-12 is the pages'
 *               threshold.
 *   stats:      device pointer or NULL.
 * Results are bitwise reproducible run to run. */
cce_status cce_backward(const void *E, const void *C, const int64_t *x,
                        const float *lse, const float *grad_loss, int64_t N,
                        int64_t V, int64_t D, int64_t ignore_index,
                        int reduction, float filter_eps, void *dE, void *dC,
                        cce_filter_stats *stats, void *workspace,
                        size_t workspace_bytes, void *stream);

/* cce_backward with a filter mode (a cce_filter_mode value; see above):
 * the same arguments, outputs, numerics and errors, plus
 * CCE_ERR_BAD_FILTER_MODE for any other value.  filter_eps applies to the
 * filtered contraction(s) only; the other one takes every unit of G.
 * stats->units_skipped counts the units left out of the filtered
 * contraction(s) (a unit counts once).  cce_backward is
 * cce_backward_ex(..., CCE_FILTER_BOTH, ...). */
cce_status cce_backward_ex(const void *E, const void *C, const int64_t *x,
                           const float *lse, const float *grad_loss, int64_t N,
                           int64_t V, int64_t D, int64_t ignore_index,
                           int reduction, float filter_eps, int filter_mode,
                           void *dE, void *dC, cce_filter_stats *stats,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/* cce_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * arguments, results and errors as cce_forward but no workspace: the
 * forward's workspace is a static device array of CCE_NOALLOC_SCRATCH_BYTES
 * inside the library, one copy per GPU it runs on, held until the process
 * ends.  The caller still owns E, C, x, loss and lse.  The call allocates
 * nothing (no hipMalloc, no library allocation); its first call on a device
 * looks up that device's copy with hipGetSymbolAddress.  Every call on one
 * GPU shares that GPU's copy, so calls that overlap on one GPU (other
 * streams, other threads) race; nothing in the array needs to be zero on
 * entry.  Shapes whose forward workspace (cce_workspace_bytes) exceeds
 * CCE_NOALLOC_SCRATCH_BYTES -- N * D * 2 bytes for the compacted copy of E
 * plus O(N) -- return CCE_ERR_SCRATCH_TOO_SMALL before anything is enqueued;
 * e.g. N = 8192 at D = 2304 needs about 37 MiB and fits, N = 16384 at
 * D = 2880 needs about 91 MiB and does not.  The array is device memory the
 * library holds on every GPU it runs on, whether or not this entry point is
 * called, so it is kept small. */
#define CCE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
cce_status cce_forward_noalloc(const void *E, const void *C, const int64_t *x,
                               int64_t N, int64_t V, int64_t D,
                               int64_t ignore_index, int reduction, float *loss,
                               float *lse, void *stream);

/* Vocabulary order ("Cut Your Losses" digest, "Vocabulary Sorting": the
 * vocabulary reordered by each entry's average logit so that the entries the
 * softmax keeps above the filter threshold share filter units, and more
 * units can be skipped).  Writes order [V] int32 (device): the vocabulary
 * ids by descending average logit a[v] = (1/N_v) sum_n C[v] . E[n] over the
 * valid rows (not ignore_index, target inside [0, V)), equal averages by
 * ascending id; a NaN average sorts last; with no valid row every average is
 * 0 and the order is the identity.  The averages are formed in fp32 as
 * C[v] . mean_n E[n] (the mean row in fp64 sums over fp32 partials), so
 * entries whose averages differ by about fp32 rounding may come in either
 * order relative to an exact computation; the result is bitwise
 * reproducible run to run.  The digest gathers the per-entry sums inside the
 * forward pass; here the order is its own call, so a caller can compute it
 * once and keep it for several steps.
 *   workspace: at least the backward's size from cce_workspace_bytes.
 * Same argument rules and errors as cce_forward. */
cce_status cce_vocab_order(const void *E, const void *C, const int64_t *x, int64_t N,
                           int64_t V, int64_t D, int64_t ignore_index, int32_t *order,
                           void *workspace, size_t workspace_bytes, void *stream);

/* cce_backward_ex with the vocabulary taken in a given order ("Cut Your
 * Losses" digest, "Vocabulary Sorting"): position i of the reordered
 * vocabulary is entry vocab_order[i].  The logits are recomputed in that
 * order, the 32 x 32 filter units are cut along it (units_total and
 * units_skipped count them so), targets follow their entries, and dC row v
 * is still the gradient of C row v.  Without the filter (filter_eps = 0) the
 * result is the unsorted backward's up to fp32 summation order.
 *   vocab_order: device, [V] int32, a permutation of 0 .. V-1 (as
 *                cce_vocab_order writes).  Entries outside [0, V) are never
 *                used as an index (their positions read as zero rows and
 *                write no dC row); any order that is not a permutation gives
 *                unspecified gradients.
 * Errors: those of cce_backward_ex; CCE_ERR_NULL_POINTER for a NULL
 * vocab_order; CCE_ERR_BAD_SHAPE also when V * D * 2 exceeds 2^31 - 16
 * bytes (the reordered rows of C are addressed by 32-bit offsets). */
cce_status cce_backward_sorted(const void *E, const void *C, const int64_t *x,
                               const float *lse, const float *grad_loss, int64_t N,
                               int64_t V, int64_t D, int64_t ignore_index,
                               int reduction, float filter_eps, int filter_mode,
                               const int32_t *vocab_order, void *dE, void *dC,
                               cce_filter_stats *stats, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *cce_status_string(cce_status status);

/* Optional per-kernel timing with HIP events recorded on the launch stream
 * around every kernel the library enqueues.  Host-side state, not thread
 * safe; meant for benchmarks.  cce_profile_enable(1) clears and starts
 * recording, cce_profile_enable(0) stops; cce_profile_enable(2) records too
 * and runs each role of the unsorted backward step in a launch of its own
 * (the same tiles and results, without the fused launch's overlap of roles),
 * reported as "bwd_de", "bwd_dc", "bwd_g" (recompute, G, filter) and "bwd_t"
 * (the scaled transpose of the C chunk) instead of "bwd_step"; other values
 * give CCE_ERR_BAD_SHAPE.  cce_profile_query synchronises on the recorded
 * events and reports, for the kernel family `name` ("fwd_lse", "target" (the
 * fp64 target logits, forward and backward), "fwd_merge", "bwd_step"
 * (recompute + G + dC + dE), "transpose", "gather" (the compacted copy of E),
 * "vocab_order", "small", or the role families above), the number of
 * launches and their summed duration in milliseconds. */
cce_status cce_profile_enable(int on);
cce_status cce_profile_query(const char *name, int64_t *launches,
                             double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* CCE_H */
