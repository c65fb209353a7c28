/*
 * bsfa.h -- C ABI of the block-sparse FlashAttention library (libbsfa.so): prefill
 * (bsfa_fwd) and decode (bsfa_decode).
 *
 * What the library computes. For every batch b, query head h (key/value head
 * g = h / (Hq / Hkv), grouped-query sharing as in the "Multi-Query and Grouped-Query
 * Attention" section of the "sparse attention mechanism" glossary page) and query row i:
 *
 *   s_ij   = scale * q_i . k_j                      ("Standard Attention Bottleneck")
 *   A(i,j) = static mask: causal AND (window OR global tokens)        (see mask spec)
 *   M_tc   = max of s_ij over the allowed elements of query tile t x key block c
 *            (64 x 64 elements)
 *   keep   = forced(t,c) OR M_tc >= tau_h            (Block Sparse Flash Attention,
 *            "The paper's summary" / "The paper's improvements": a calibrated
 *            per-head threshold on each block's maximum; blocks below it are skipped)
 *   K_i    = { j : A(i,j) and keep(i/64, j/64) }     (the index set G of the page
 *            "Sparse attention weights assumption", "Sparse Attention Output Formula")
 *   LSE_i  = log sum_{j in K_i} exp(s_ij);   O_i = sum_{j in K_i} exp(s_ij - LSE_i) v_j
 *
 * Skipped blocks leave both the numerator and the denominator of the softmax (the kept
 * weights are renormalised), and their V block is never read. A row with an empty K_i
 * gets O_i = 0 and LSE_i = -inf. The tiles are processed FlashAttention-style with a
 * running max and sum ("sparse attention mechanism" glossary, "FlashAttention"), so no
 * N x N matrix exists anywhere.
 *
 * Conventions for every entry point:
 * - All functions are thread-safe, allocate no device memory and keep no per-call state.
 * - Buffers are owned by the caller. "device" means HIP device memory on the current
 *   device; "host" means ordinary host memory.
 * - Return value: BSFA_OK (0) or a negative bsfa_status. On failure
 *   bsfa_last_error() returns a thread-local message. Argument checks happen before any
 *   work is queued, so a failed call has no side effects.
 * - Kernel faults are asynchronous: they surface at the caller's next synchronisation.
 */
#ifndef BSFA_H
#define BSFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSFA_OK = 0,
  BSFA_ERR_INVALID_ARG = -1,      /* null pointer, negative size, inconsistent shapes   */
  BSFA_ERR_UNSUPPORTED = -2,      /* valid but not implemented (head dim, alignment)    */
  BSFA_ERR_BUFFER_TOO_SMALL = -3, /* a caller buffer (block lists, workspace) too small */
  BSFA_ERR_HIP = -4               /* a HIP runtime call failed; message has the reason  */
} bsfa_status;

typedef enum { BSFA_OUT_BF16 = 0, BSFA_OUT_F32 = 1 } bsfa_out_dtype;

/* Block classes (bit flags in bsfa_block_lists.cls). */
#define BSFA_CLS_PARTIAL 1u /* some element of the 64x64 tile is masked: test per element */
#define BSFA_CLS_FORCED 2u  /* the gate never skips this tile                              */
#define BSFA_CLS_RANDOM 4u  /* the random primitive selects this tile's 64-token blocks    */

/*
 * Static sparsity primitives, OR-composed as in "SAS: Sparse Attention Synthesizer",
 * Step 5 (Logic Operators), with the patterns of the "sparse attention mechanism"
 * glossary (table "Sparse Attention Patterns"). Element (i, j), 0-based, 0 <= i, j < N,
 * is allowed iff
 *   (!causal || j <= i) && (no pattern primitive set || pattern(i, j))
 * where pattern(i, j) is the OR of the primitives that are set:
 *   window > 0        |i - j| < window   (causal: the glossary's "Mistral/Mixtral
 *                     Sliding Window Attention" range [max(0, i - W + 1), i])
 *   dilation > 0      (i - j) is a multiple of dilation ("every k-th token"), and, when
 *                     dilation_taps > 0, |i - j| < dilation * dilation_taps
 *   block > 0         i / block == j / block ("attend within fixed-size blocks")
 *   random_ppm > 0    the 64-token blocks (i / 64, j / 64) are chosen by the random
 *                     primitive (BigBird's random attention): SplitMix64 of the counter
 *                     (random_seed mod 2^24) * 2^40 + (i / 64) * 2^20 + (j / 64), kept
 *                     when its top 32 bits are below floor(random_ppm * 2^32 / 10^6)
 *   n_global > 0      j < n_global or i < n_global ("Global Tokens in Attention": the
 *                     first tokens are visible to all, and see all); with no other
 *                     primitive set this changes nothing
 * Forcing: the tile holding a diagonal element (i, i) is never skipped when
 * force_keep_diag != 0, and tiles holding a key j < n_global are never skipped when
 * force_keep_global != 0. Field limits: window, n_global, dilation, dilation_taps,
 * block >= 0; 0 <= random_ppm <= 1000000; random_seed any.
 */
typedef struct {
  int32_t causal;
  int32_t window;
  int32_t n_global;
  int32_t force_keep_diag;
  int32_t force_keep_global;
  int32_t dilation;
  int32_t dilation_taps;
  int32_t block;
  int32_t random_ppm;
  int32_t random_seed;
} bsfa_mask_spec;

/* Element strides of a [B, H, N, d] tensor; the d dimension must be contiguous. */
typedef struct {
  int64_t b, h, n;
} bsfa_strides;

/*
 * Static block lists in CSR form, shared by every batch entry and head: query tile t
 * owns entries [row_ptr[t], row_ptr[t+1]), each a key block index col[e] (ascending)
 * and a class cls[e] (BSFA_CLS_* flags). Tiles with no allowed element are absent.
 * For bsfa_fwd the three arrays are in device memory and must come from
 * bsfa_build_block_lists for the same mask spec, N and 64x64 blocks. Each array must be
 * 4-byte aligned, and cls must stay readable up to the next 4-byte boundary past its
 * last entry (the kernel reads it as aligned 32-bit words; any hipMalloc allocation
 * satisfies this).
 */
typedef struct {
  int32_t n_qtiles; /* ceil(N / block_q)                    */
  int32_t block_q;  /* must be 64 for bsfa_fwd              */
  int32_t block_k;  /* must be 64 for bsfa_fwd              */
  int64_t nnz;      /* entries in col / cls                 */
  const int32_t* row_ptr; /* [n_qtiles + 1] */
  const int32_t* col;     /* [nnz]          */
  const uint8_t* cls;     /* [nnz]          */
} bsfa_block_lists;

/*
 * Build the static block lists on the host (pure CPU; no HIP call).
 *   mask            : static pattern (host).
 *   N               : sequence length, N >= 0 (N need not be a multiple of the block).
 *   block_q, block_k: tile sizes, >= 1.
 *   row_ptr         : host [ceil(N/block_q) + 1], always written (may be NULL to only
 *                     size the lists).
 *   col, cls        : host [capacity]; if col == NULL only *nnz_out is computed
 *                     (two-call sizing).
 *   nnz_out         : host, receives the number of entries. Required.
 * Returns BSFA_ERR_BUFFER_TOO_SMALL (with *nnz_out set) when capacity < nnz.
 * A tile is PARTIAL when any of its block_q x block_k element slots (including slots
 * past N in a ragged last tile) is not allowed; FORCED follows the mask spec's flags.
 */
int bsfa_build_block_lists(const bsfa_mask_spec* mask, int32_t N, int32_t block_q,
                           int32_t block_k, int32_t* row_ptr, int32_t* col, uint8_t* cls,
                           int64_t capacity, int64_t* nnz_out);

/*
 * Block-sparse FlashAttention forward (prefill) on the GPU, queued on `stream`.
 *   q   : device bf16 [B, Hq, N, d] with strides *sq (elements).
 *   k, v: device bf16 [B, Hkv, N, d] with strides *sk, *sv. Hq % Hkv == 0.
 *   out : device [B, Hq, N, d], bf16 or fp32 (out_dtype), strides *so.
 *   lse : device fp32 [B, Hq, N] contiguous (natural log); may be NULL.
 *   d   : 64 or 128. N >= 0 (any N; ragged last tiles are masked). B, Hq, Hkv >= 1.
 *   mask, lists: the static pattern and its device block lists (see above).
 *   tau : device fp32 [Hq], thresholds in scaled-score units (same units as s_ij);
 *         NULL selects the dense path (every allowed tile kept, no gate evaluated).
 *         tau = -inf keeps every tile through the gated path; NaN keeps forced tiles only.
 *   softmax_scale: the scale in s_ij; 0 selects 1/sqrt(d).
 *   stats   : device uint64 [B*Hq*2] = {kept, skipped} tile counts per (b, h); counts
 *             are ADDED to the buffer (zero it first); may be NULL.
 *   tile_max, keep: device fp32 / uint8 [B*Hq*lists->nnz], per (b, h, CSR entry) the
 *             block maximum M_tc and the keep decision; both NULL or both set; needs
 *             tau != NULL.
 *   stream  : hipStream_t (NULL = default stream). The call is asynchronous.
 * Pointers q, k, v, out must be 16-byte aligned and the n/h/b strides non-negative
 * multiples of 8. The K (and V) rows of one (batch, KV head), ((N - 1) * n-stride + d)
 * elements, must span fewer than 2^31 bytes; otherwise BSFA_ERR_UNSUPPORTED. So is a
 * launch of 2^32 or more work-items. A workgroup of 512 work-items serves four (query
 * head, 64-row query tile) pairs of one KV head: P heads of 4 / P adjacent query tiles,
 * P = 4, 2 or 1 as Hq / Hkv is a multiple of 4, even, or odd. So
 * B * (Hq / P) * ceil(ceil(N / 64) / (4 / P)) * 512 must stay below 2^32, and for P < 4
 * (the workgroup counts the union of its tiles' block lists in a 64 KiB LDS bitmap)
 * ceil(N / 64) must stay below 524288.
 */
int bsfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
             const bsfa_strides* sq, const bsfa_strides* sk, const bsfa_strides* sv,
             const bsfa_strides* so, const bsfa_mask_spec* mask,
             const bsfa_block_lists* lists, const float* tau, float softmax_scale,
             int32_t out_dtype, uint64_t* stats, float* tile_max, uint8_t* keep,
             void* stream);

/*
 * Decode (token generation): one new query row per sequence b and query head h against
 * a key/value cache. Token generation adds one token at a time and attends over the
 * cached keys and values of all earlier tokens ("SAS: Sparse Attention Synthesizer",
 * Challenge 2 "KV Cache Management" and Step 6). The gate is the one of bsfa_fwd with the
 * single row as the query tile:
 *   n      = min(lengths[b], max_len) valid cache rows; the row is the newest token,
 *            position i = n - 1, whose own key and value are already cached
 *   s_j    = scale * q . k_j for cached keys j < n; A(i, j) the static mask at row i
 *   M_c    = max of s_j over the allowed keys of 64-key block c
 *   keep_c = forced(c) OR M_c >= tau_h, forced(c): c holds key i (force_keep_diag) or a
 *            key j < n_global (force_keep_global)
 *   LSE    = log sum_{kept j} exp(s_j);  O = sum_{kept j} exp(s_j - LSE) v_j
 * A V block is read only when some query head of its KV group keeps it. A row with no
 * kept key (lengths[b] <= 0) gets O = 0 and LSE = -inf. Cache rows at or past n are never
 * read (they may hold anything).
 *
 * The cache is split into groups of 4 blocks (256 keys); each (sequence, KV head, split)
 * writes a partial (O_s, LSE_s) per head into the caller's workspace, and a second
 * kernel merges them (LSE = log sum_s exp LSE_s, O = sum_s exp(LSE_s - LSE) O_s).
 */

/* Workspace bytes bsfa_decode needs: B * Hq * ceil(ceil(max_len / 64) / 4) * (d + 4) * 4.
 * B >= 0, Hq >= 1, max_len >= 1, d in {64, 128}. */
int bsfa_decode_workspace_size(int32_t B, int32_t Hq, int32_t max_len, int32_t d,
                               int64_t* bytes);

/*
 * One decode step on the GPU, queued on `stream`.
 *   q       : device bf16 [B, Hq, d]; row (b, h) at q + b * sq->b + h * sq->h (sq->n unused).
 *   k_cache, v_cache: device bf16 [B, Hkv, max_len, d] with strides *sk, *sv. Hq % Hkv == 0
 *             and Hq / Hkv <= 32.
 *   lengths : device int32 [B], valid cache rows per sequence (values above max_len count
 *             as max_len, values <= 0 as no rows). 4-byte aligned.
 *   out     : device [B, Hq, d], bf16 or fp32 (out_dtype), strides *so (so->n unused).
 *   lse     : device fp32 [B * Hq] (natural log); may be NULL.
 *   max_len : cache rows, >= 1. d: 64 or 128.
 *   mask    : static pattern (as for bsfa_fwd), evaluated at row i = n - 1.
 *   tau     : device fp32 [Hq] in scaled-score units; NULL selects the dense path (every
 *             allowed block kept). NaN keeps forced blocks only.
 *   softmax_scale: 0 selects 1/sqrt(d).
 *   stats   : device uint64 [B*Hq*2] = {kept, skipped} allowed blocks per (b, h), ADDED to
 *             the buffer; may be NULL.
 *   tile_max, keep: device fp32 / uint8 [B*Hq*nkb], nkb = ceil(max_len / 64): per (b, h,
 *             block c) M_c (-inf where no key of the block is allowed or c >= ceil(n/64))
 *             and the keep bit; both NULL or both set; needs tau != NULL.
 *   workspace, workspace_bytes: device scratch of at least bsfa_decode_workspace_size
 *             bytes, 16-byte aligned; its contents on entry do not matter. Calls that
 *             share one workspace must not overlap in time.
 * Pointers q, k_cache, v_cache, out must be 16-byte aligned and the used strides
 * non-negative multiples of 8; the cache rows of one (sequence, KV head),
 * ((max_len - 1) * n-stride + d) elements, must span fewer than 2^31 bytes.
 * Errors: BSFA_ERR_BUFFER_TOO_SMALL for a short workspace, otherwise as bsfa_fwd; the
 * work-item limit applies to B * Hkv * ceil(ceil(max_len / 64) / 4) * 128 and to
 * B * Hq * (d / 32) * 256.
 */
int bsfa_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* lengths, void* out, float* lse, int32_t B, int32_t Hq,
                int32_t Hkv, int32_t max_len, int32_t d, const bsfa_strides* sq,
                const bsfa_strides* sk, const bsfa_strides* sv, const bsfa_strides* so,
                const bsfa_mask_spec* mask, const float* tau, float softmax_scale,
                int32_t out_dtype, uint64_t* stats, float* tile_max, uint8_t* keep,
                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * bsfa_decode_static: bsfa_decode without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc). The per-split partials that bsfa_decode keeps in the caller's
 * workspace live instead in a fixed device array inside the library,
 * BSFA_DECODE_STATIC_SCRATCH_BYTES (32 MiB) on every GPU the library runs on, held until
 * the process ends. The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the array's device address is looked up once per device,
 * on the first call for that device.
 *   Arguments, layouts, ownership and results: as bsfa_decode, without workspace and
 *   workspace_bytes. The launch goes to the device of `stream` (NULL: the current device).
 * Errors: as bsfa_decode; a step that needs more scratch than the array holds
 * (bsfa_decode_workspace_size above BSFA_DECODE_STATIC_SCRATCH_BYTES) returns
 * BSFA_ERR_BUFFER_TOO_SMALL before any work is queued.
 * Concurrency: every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs clearing: each call writes the partials it reads). Calls
 * that overlap in time on one GPU (on different streams or host threads) race and give
 * wrong results: the caller serialises them, e.g. on one stream.
 */
#define BSFA_DECODE_STATIC_SCRATCH_BYTES (32ll * 1024 * 1024)
int bsfa_decode_static(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* lengths, void* out, float* lse, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t max_len, int32_t d, const bsfa_strides* sq,
                       const bsfa_strides* sk, const bsfa_strides* sv,
                       const bsfa_strides* so, const bsfa_mask_spec* mask, const float* tau,
                       float softmax_scale, int32_t out_dtype, uint64_t* stats,
                       float* tile_max, uint8_t* keep, void* stream);

/*
 * Per-head threshold calibration on the GPU. Thresholds are learned once per layer and
 * head from the distribution of block maxima on calibration data (Block Sparse Flash
 * Attention, "The paper's improvements"); here tau_h is the `quantile` of head h's
 * eligible block maxima with numpy's default linear interpolation, computed in fp64 and
 * rounded to fp32. It equals np.quantile over the same maxima.
 *   tile_max, keep: device fp32 / uint8 [B, Hq, n_blocks], the per-block export of one
 *             gate-only pass (bsfa_fwd with tau = NaN and lists->nnz blocks per (b, h), or
 *             bsfa_decode with tau = NaN and ceil(max_len / 64) blocks). A block is
 *             eligible when keep is 0 (not forced) and its maximum is finite (allowed).
 *   quantile: in [0, 1].
 *   tau     : device fp32 [Hq], written; -inf for a head with no eligible block.
 *   workspace, workspace_bytes: device scratch of at least
 *             bsfa_calibrate_workspace_size(Hq) bytes, 16-byte aligned; its contents on
 *             entry do not matter. Calls that share one workspace must not overlap.
 *   stream  : hipStream_t; the call is asynchronous (ten small kernels).
 * Errors: INVALID_ARG for negative sizes, a quantile outside [0, 1] or NaN, or missing
 * pointers; BUFFER_TOO_SMALL for a short workspace; UNSUPPORTED for misaligned pointers,
 * 2^32 - 1 or more blocks per head, or a dispatch of 2^32 or more work-items.
 */
int bsfa_calibrate_workspace_size(int32_t Hq, int64_t* bytes);
int bsfa_calibrate_tau(const float* tile_max, const uint8_t* keep, int32_t B, int32_t Hq,
                       int64_t n_blocks, double quantile, float* tau, void* workspace,
                       int64_t workspace_bytes, void* stream);

/*
 * Copy the per-(b, h) counters written by bsfa_fwd or bsfa_decode to the host and split
 * them.
 *   stats_dev: device uint64 [B*Hq*2]; kept_host, skipped_host: host uint64 [B*Hq].
 * Synchronises `stream` before returning.
 */
int bsfa_skip_stats(const uint64_t* stats_dev, int32_t B, int32_t Hq, uint64_t* kept_host,
                    uint64_t* skipped_host, void* stream);

/* Thread-local text for the last failing call on this thread ("" if none). */
const char* bsfa_last_error(void);

/* Library ABI version (this header: 5). */
int32_t bsfa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSFA_H */
