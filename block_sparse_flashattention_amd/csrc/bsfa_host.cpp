// Host side of libbsfa: static block lists, argument validation, variant dispatch.
//
// Block classification is analytic per tile (no per-element loop): the static mask is
// causal AND (window band OR global key OR global query), so "some element allowed"
// and "every element allowed" reduce to interval tests on the tile's row and column
// ranges.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/bsfa.h"
#include "bsfa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return BSFA_OK;
}

// Rows [r0, r1] and columns [c0, c1] (inclusive, already clipped to [0, N-1]).
bool any_allowed(const bsfa_mask_spec& m, int64_t r0, int64_t r1, int64_t c0, int64_t c1) {
  if (m.window <= 0) return !m.causal || c0 <= r1;
  const int64_t ng = m.n_global;
  if (ng > 0 && c0 < ng && (!m.causal || c0 <= r1)) return true;        // global key
  if (ng > 0 && r0 < ng && (!m.causal || c0 <= std::min(r1, ng - 1))) return true;  // global query
  // band |i - j| < W: the differences i - j cover every integer in [r0 - c1, r1 - c0]
  int64_t lo = r0 - c1, hi = r1 - c0;
  lo = std::max<int64_t>(lo, m.causal ? 0 : -(int64_t)(m.window - 1));
  hi = std::min<int64_t>(hi, m.window - 1);
  return lo <= hi;
}

bool all_allowed(const bsfa_mask_spec& m, int64_t r0, int64_t r1, int64_t c0, int64_t c1) {
  if (m.causal && c1 > r0) return false;
  if (m.window <= 0) return true;
  const int64_t ng = m.n_global;
  // pairs not rescued by a global row or column must lie in the band
  const int64_t rr0 = std::max(r0, ng), cc0 = std::max(c0, ng);
  if (rr0 > r1 || cc0 > c1) return true;
  return std::max(r1 - cc0, c1 - rr0) < m.window;
}

bool valid_strides(const bsfa_strides* s) {
  return s && s->b % 8 == 0 && s->h % 8 == 0 && s->n % 8 == 0 && s->b >= 0 && s->h >= 0 &&
         s->n >= 0;
}

// K and V rows of one (batch, KV head) are read through a buffer view with a 32-bit
// byte range: the view must span less than 2^31 bytes.
bool view_fits(const bsfa_strides* s, int32_t N, int32_t d) {
  return ((int64_t)(N - 1) * s->n + d) * 2 <= (int64_t)INT32_MAX;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* bsfa_last_error(void) { return g_last_error.c_str(); }

int32_t bsfa_abi_version(void) { return 1; }

int bsfa_build_block_lists(const bsfa_mask_spec* mask, int32_t N, int32_t block_q,
                           int32_t block_k, int32_t* row_ptr, int32_t* col, uint8_t* cls,
                           int64_t capacity, int64_t* nnz_out) {
  if (!mask || !nnz_out) return fail(BSFA_ERR_INVALID_ARG, "mask and nnz_out are required");
  if (N < 0 || block_q < 1 || block_k < 1)
    return fail(BSFA_ERR_INVALID_ARG, "need N >= 0 and block sizes >= 1 (N=%d bq=%d bk=%d)",
                N, block_q, block_k);
  if (mask->window < 0 || mask->n_global < 0)
    return fail(BSFA_ERR_INVALID_ARG, "window and n_global must be >= 0");
  if (col && !cls) return fail(BSFA_ERR_INVALID_ARG, "col and cls must both be given");
  const int64_t nqt = ((int64_t)N + block_q - 1) / block_q;
  const int64_t nkb = ((int64_t)N + block_k - 1) / block_k;
  int64_t nnz = 0;
  bool overflow = false;
  if (row_ptr) row_ptr[0] = 0;
  for (int64_t t = 0; t < nqt; ++t) {
    const int64_t r0 = t * block_q, r1 = std::min<int64_t>(r0 + block_q, N) - 1;
    const bool rows_whole = r0 + block_q <= N;
    for (int64_t c = 0; c < nkb; ++c) {
      const int64_t c0 = c * block_k, c1 = std::min<int64_t>(c0 + block_k, N) - 1;
      if (!any_allowed(*mask, r0, r1, c0, c1)) continue;
      if (col) {
        if (nnz < capacity) {
          const bool whole = rows_whole && c0 + block_k <= N;
          uint8_t k = 0;
          if (!(whole && all_allowed(*mask, r0, r1, c0, c1))) k |= BSFA_CLS_PARTIAL;
          const bool diag = std::max(r0, c0) <= std::min(r1, c1);
          const bool glob = c0 < std::min<int64_t>(mask->n_global, N);
          if ((mask->force_keep_diag && diag) || (mask->force_keep_global && glob))
            k |= BSFA_CLS_FORCED;
          col[nnz] = (int32_t)c;
          cls[nnz] = k;
        } else {
          overflow = true;
        }
      }
      ++nnz;
    }
    if (row_ptr) {
      if (nnz > INT32_MAX) return fail(BSFA_ERR_UNSUPPORTED, "more than 2^31 - 1 tiles");
      row_ptr[t + 1] = (int32_t)nnz;
    }
  }
  *nnz_out = nnz;
  if (overflow)
    return fail(BSFA_ERR_BUFFER_TOO_SMALL, "capacity %lld < %lld entries", (long long)capacity,
                (long long)nnz);
  return ok();
}

int bsfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int32_t B,
             int32_t Hq, int32_t Hkv, int32_t N, int32_t d, const bsfa_strides* sq,
             const bsfa_strides* sk, const bsfa_strides* sv, const bsfa_strides* so,
             const bsfa_mask_spec* mask, const bsfa_block_lists* lists, const float* tau,
             float softmax_scale, int32_t out_dtype, uint64_t* stats, float* tile_max,
             uint8_t* keep, void* stream) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1)
    return fail(BSFA_ERR_INVALID_ARG, "need B >= 0, N >= 0, Hq >= 1, Hkv >= 1");
  if (Hq % Hkv != 0) return fail(BSFA_ERR_INVALID_ARG, "Hq (%d) %% Hkv (%d) != 0", Hq, Hkv);
  if (!mask || !lists) return fail(BSFA_ERR_INVALID_ARG, "mask and lists are required");
  if (out_dtype != BSFA_OUT_BF16 && out_dtype != BSFA_OUT_F32)
    return fail(BSFA_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale))
    return fail(BSFA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if ((tile_max == nullptr) != (keep == nullptr))
    return fail(BSFA_ERR_INVALID_ARG, "tile_max and keep must be given together");
  if (tile_max && !tau)
    return fail(BSFA_ERR_INVALID_ARG, "the per-tile export needs tau (the gated path)");
  if (d != 64 && d != 128) return fail(BSFA_ERR_UNSUPPORTED, "head dim %d (need 64 or 128)", d);
  if (lists->block_q != 64 || lists->block_k != 64)
    return fail(BSFA_ERR_UNSUPPORTED, "block lists must use 64x64 tiles");
  const int32_t nqt = (N + 63) / 64;
  if (lists->n_qtiles != nqt)
    return fail(BSFA_ERR_INVALID_ARG, "lists have %d query tiles, N=%d needs %d",
                lists->n_qtiles, N, nqt);
  if (lists->nnz < 0) return fail(BSFA_ERR_INVALID_ARG, "lists->nnz < 0");
  if (B == 0 || N == 0) return ok();  // nothing to compute
  if (!q || !k || !v || !out) return fail(BSFA_ERR_INVALID_ARG, "q, k, v, out are required");
  if (!lists->row_ptr || (lists->nnz > 0 && (!lists->col || !lists->cls)))
    return fail(BSFA_ERR_INVALID_ARG, "block list arrays missing");
  if (((uintptr_t)lists->row_ptr | (uintptr_t)lists->col | (uintptr_t)lists->cls) & 3u)
    return fail(BSFA_ERR_UNSUPPORTED, "block list arrays must be 4-byte aligned");
  if (!sq || !sk || !sv || !so) return fail(BSFA_ERR_INVALID_ARG, "strides are required");
  if (!valid_strides(sq) || !valid_strides(sk) || !valid_strides(sv) || !valid_strides(so))
    return fail(BSFA_ERR_UNSUPPORTED, "strides must be non-negative multiples of 8 elements");
  if (!view_fits(sk, N, d) || !view_fits(sv, N, d))
    return fail(BSFA_ERR_UNSUPPORTED, "the K or V rows of one head span 2^31 bytes or more");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(BSFA_ERR_UNSUPPORTED, "q, k, v, out must be 16-byte aligned");

  const int group = Hq / Hkv;
  const int hpack = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  const int64_t grid = (int64_t)B * (Hq / hpack) * nqt;
  if (grid > INT32_MAX) return fail(BSFA_ERR_UNSUPPORTED, "grid too large");

  bsfa::FwdArgs a;
  memset(&a, 0, sizeof a);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = out;
  a.lse = lse;
  a.sqb = sq->b; a.sqh = sq->h; a.sqn = sq->n;
  a.skb = sk->b; a.skh = sk->h; a.skn = sk->n;
  a.svb = sv->b; a.svh = sv->h; a.svn = sv->n;
  a.sob = so->b; a.soh = so->h; a.son = so->n;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N;
  a.nqt = nqt;
  a.group = group;
  a.causal = mask->causal != 0;
  a.window = mask->window;
  a.n_global = mask->n_global;
  a.row_ptr = lists->row_ptr;
  a.col = lists->col;
  a.cls = lists->cls;
  a.nnz = lists->nnz;
  a.tau = tau;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.stats = (unsigned long long*)stats;
  a.tile_max = tile_max;
  a.keep = keep;
  const char* err = nullptr;
  int rc = bsfa::launch_fwd(a, d, hpack, out_dtype == BSFA_OUT_F32, stream, &err);
  if (rc != BSFA_OK) return fail(rc, "%s", err ? err : "launch failed");
  return ok();
}

int bsfa_skip_stats(const uint64_t* stats_dev, int32_t B, int32_t Hq, uint64_t* kept_host,
                    uint64_t* skipped_host, void* stream) {
  if (!stats_dev || !kept_host || !skipped_host)
    return fail(BSFA_ERR_INVALID_ARG, "stats_dev, kept_host and skipped_host are required");
  if (B < 0 || Hq < 1) return fail(BSFA_ERR_INVALID_ARG, "need B >= 0 and Hq >= 1");
  const size_t n = (size_t)B * (size_t)Hq;
  if (n == 0) return ok();
  uint64_t* both = new uint64_t[2 * n];
  const char* err = nullptr;
  const int rc = bsfa::copy_to_host_sync(both, stats_dev, 2 * n * sizeof(uint64_t), stream, &err);
  if (rc == BSFA_OK) {
    for (size_t i = 0; i < n; ++i) {
      kept_host[i] = both[2 * i];
      skipped_host[i] = both[2 * i + 1];
    }
  }
  delete[] both;
  if (rc != BSFA_OK) return fail(rc, "%s", err ? err : "copy failed");
  return ok();
}

}  // extern "C"
