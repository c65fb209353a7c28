// Host side of libbsfa: static block lists, argument validation, variant dispatch.
//
// Block classification. With only the causal, window and global primitives it is
// analytic per tile: "some element allowed" and "every element allowed" reduce to
// interval tests on the tile's row and column ranges. With the dilated, blockwise or
// random primitives, a conservative per-primitive test first discards tiles no
// primitive can reach; the remaining tiles are classified exactly from per-row 64-bit
// masks of their allowed keys.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
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

bool extra_primitives(const bsfa_mask_spec& m) {
  return m.dilation > 0 || m.block > 0 || m.random_ppm > 0;
}
bool has_pattern(const bsfa_mask_spec& m) { return m.window > 0 || extra_primitives(m); }

int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// SplitMix64 output for counter x (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014).
uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The random primitive's choice for 64-token query block t and key block c.
bool random_block(const bsfa_mask_spec& m, int64_t t, int64_t c) {
  if (m.random_ppm <= 0) return false;
  const uint64_t counter = ((uint64_t)((uint32_t)m.random_seed & 0xFFFFFFu) << 40) |
                           ((uint64_t)(t & 0xFFFFF) << 20) | (uint64_t)(c & 0xFFFFF);
  const uint64_t threshold = ((uint64_t)m.random_ppm << 32) / 1000000u;
  return (splitmix64(counter) >> 32) < threshold;
}

// Bits [0, n) of a 64-bit word, n clamped to [0, 64].
uint64_t bits_below(int64_t n) {
  if (n <= 0) return 0;
  if (n >= 64) return ~0ull;
  return (1ull << n) - 1ull;
}

// Bits at 0, s, 2s, ... below 64 (the dilated primitive's pattern for one residue).
uint64_t stride_pattern(int32_t s) {
  if (s <= 0) return 0;
  uint64_t p = 0;
  for (int k = 0; k < 64; k += s) p |= 1ull << k;
  return p;
}

// Keys j0 + k (k in [0, 64)) that query row i may attend, as bit k.
uint64_t row_bits(const bsfa_mask_spec& m, int64_t i, int64_t j0, int64_t N,
                  uint64_t spat) {
  if (i < 0 || i >= N) return 0;
  const int64_t r = i - j0;  // k of the diagonal element
  uint64_t mm = bits_below(N - j0);
  if (m.causal) mm &= bits_below(r + 1);
  if (!has_pattern(m)) return mm;
  uint64_t p = (i < m.n_global) ? ~0ull : bits_below((int64_t)m.n_global - j0);
  if (m.window > 0) p |= bits_below(r + m.window) & ~bits_below(r - m.window + 1);
  if (m.dilation > 0) {
    const int64_t st = m.dilation;
    const int64_t off = ((r % st) + st) % st;
    uint64_t dm = 0;
    if (off < 64) dm = (st >= 64 ? 1ull : spat) << off;
    if (m.dilation_taps > 0) {
      const int64_t span = st * (int64_t)m.dilation_taps;
      dm &= bits_below(r + span) & ~bits_below(r - span + 1);
    }
    p |= dm;
  }
  if (m.block > 0) {
    const int64_t lo = (i / m.block) * (int64_t)m.block;
    p |= bits_below(lo + m.block - j0) & ~bits_below(lo - j0);
  }
  if (m.random_ppm > 0) {  // the 64 keys may straddle two 64-token blocks
    const int64_t cb = floor_div(j0, 64), split = (cb + 1) * 64 - j0;
    const uint64_t low = bits_below(split);
    if (random_block(m, i / 64, cb)) p |= low;
    if (split < 64 && random_block(m, i / 64, cb + 1)) p |= ~low;
  }
  return mm & p;
}

// Can any primitive reach rows [r0, r1] x columns [c0, c1]? (May say yes wrongly,
// never no wrongly.)
bool may_hit(const bsfa_mask_spec& m, int64_t r0, int64_t r1, int64_t c0, int64_t c1) {
  if (m.causal && c0 > r1) return false;
  if (!has_pattern(m)) return true;
  if (c0 < m.n_global || r0 < m.n_global) return true;
  const int64_t dlo = m.causal ? std::max<int64_t>(r0 - c1, 0) : r0 - c1, dhi = r1 - c0;
  if (m.window > 0 && std::max<int64_t>(dlo, -(int64_t)m.window + 1) <=
                          std::min<int64_t>(dhi, m.window - 1))
    return true;
  if (m.dilation > 0) {
    int64_t lo = dlo, hi = dhi;
    if (m.dilation_taps > 0) {
      const int64_t span = (int64_t)m.dilation * m.dilation_taps;
      lo = std::max(lo, -span + 1);
      hi = std::min(hi, span - 1);
    }
    if (lo <= hi && floor_div(hi, m.dilation) * m.dilation >= lo) return true;
  }
  if (m.block > 0 && std::max(r0 / m.block, c0 / m.block) <= std::min(r1 / m.block, c1 / m.block))
    return true;
  if (m.random_ppm > 0)
    for (int64_t t = r0 / 64; t <= r1 / 64; ++t)
      for (int64_t c = c0 / 64; c <= c1 / 64; ++c)
        if (random_block(m, t, c)) return true;
  return false;
}

// Exact "some element allowed" and "every element slot allowed" of a tile from its rows'
// key masks. Slots past N count as not allowed.
void classify_rows(const bsfa_mask_spec& m, int64_t r0, int64_t r1, int64_t c0, int64_t c1,
                   int64_t bq, int64_t bk, int64_t N, uint64_t spat, bool& any, bool& all) {
  any = false;
  all = (r1 - r0 + 1 == bq) && (c1 - c0 + 1 == bk);
  for (int64_t i = r0; i <= r1; ++i) {
    for (int64_t j0 = c0; j0 <= c1; j0 += 64) {
      const uint64_t width = bits_below(std::min<int64_t>(64, c1 - j0 + 1));
      const uint64_t mm = row_bits(m, i, j0, N, spat) & width;
      any = any || mm != 0;
      all = all && mm == width;
      if (any && !all) return;
    }
  }
}

bool valid_mask(const bsfa_mask_spec* m) {
  return m->window >= 0 && m->n_global >= 0 && m->dilation >= 0 && m->dilation_taps >= 0 &&
         m->block >= 0 && m->random_ppm >= 0 && m->random_ppm <= 1000000;
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

// Calibration workspace: the per-head digit histograms, then the per-head select states.
int64_t calib_workspace_bytes(int32_t Hq) {
  return (int64_t)Hq * 256 * (int64_t)sizeof(uint32_t) +
         (int64_t)Hq * (int64_t)sizeof(bsfa::CalibState);
}

// Decode splits: one workgroup per bsfa::DEC_BPS key blocks of the cache.
int32_t decode_splits(int32_t max_len) {
  const int32_t nkb = (max_len + 63) / 64;
  return (nkb + bsfa::DEC_BPS - 1) / bsfa::DEC_BPS;
}

}  // namespace

extern "C" {

const char* bsfa_last_error(void) { return g_last_error.c_str(); }

int32_t bsfa_abi_version(void) { return 5; }

int bsfa_build_block_lists(const bsfa_mask_spec* mask, int32_t N, int32_t block_q,
                           int32_t block_k, int32_t* row_ptr, int32_t* col, uint8_t* cls,
                           int64_t capacity, int64_t* nnz_out) {
  if (!mask || !nnz_out) return fail(BSFA_ERR_INVALID_ARG, "mask and nnz_out are required");
  if (N < 0 || block_q < 1 || block_k < 1)
    return fail(BSFA_ERR_INVALID_ARG, "need N >= 0 and block sizes >= 1 (N=%d bq=%d bk=%d)",
                N, block_q, block_k);
  if (!valid_mask(mask))
    return fail(BSFA_ERR_INVALID_ARG,
                "mask fields must be >= 0 and random_ppm at most 1000000");
  if (col && !cls) return fail(BSFA_ERR_INVALID_ARG, "col and cls must both be given");
  const int64_t nqt = ((int64_t)N + block_q - 1) / block_q;
  const int64_t nkb = ((int64_t)N + block_k - 1) / block_k;
  int64_t nnz = 0;
  bool overflow = false;
  if (row_ptr) row_ptr[0] = 0;
  const bool general = extra_primitives(*mask);
  const uint64_t spat = stride_pattern(mask->dilation);
  for (int64_t t = 0; t < nqt; ++t) {
    const int64_t r0 = t * block_q, r1 = std::min<int64_t>(r0 + block_q, N) - 1;
    const bool rows_whole = r0 + block_q <= N;
    for (int64_t c = 0; c < nkb; ++c) {
      const int64_t c0 = c * block_k, c1 = std::min<int64_t>(c0 + block_k, N) - 1;
      bool any, all;
      if (general) {
        if (!may_hit(*mask, r0, r1, c0, c1)) continue;
        classify_rows(*mask, r0, r1, c0, c1, block_q, block_k, N, spat, any, all);
        if (!any) continue;
      } else {
        if (!any_allowed(*mask, r0, r1, c0, c1)) continue;
        any = true;
        all = rows_whole && c0 + block_k <= N && all_allowed(*mask, r0, r1, c0, c1);
      }
      if (col) {
        if (nnz < capacity) {
          uint8_t k = 0;
          if (!all) k |= BSFA_CLS_PARTIAL;
          const bool diag = std::max(r0, c0) <= std::min(r1, c1);
          const bool glob = c0 < std::min<int64_t>(mask->n_global, N);
          if ((mask->force_keep_diag && diag) || (mask->force_keep_global && glob))
            k |= BSFA_CLS_FORCED;
          if (mask->random_ppm > 0 && random_block(*mask, r0 / 64, c0 / 64))
            k |= BSFA_CLS_RANDOM;
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
  if (!valid_mask(mask))
    return fail(BSFA_ERR_INVALID_ARG,
                "mask fields must be >= 0 and random_ppm at most 1000000");
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
  // heads per workgroup; the workgroup's four members are hpack heads of 4 / hpack query
  // tiles
  const int hpack = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  const int tq = 4 / hpack;
  const int64_t grid = (int64_t)B * (Hq / hpack) * ((nqt + tq - 1) / tq);
  // one dispatch counts its work-items in 32 bits
  const int64_t wg_threads = 512;
  if (grid * wg_threads > (int64_t)UINT32_MAX)
    return fail(BSFA_ERR_UNSUPPORTED, "grid of %lld workgroups too large", (long long)grid);
  // workgroups of several query tiles count their steps in a bitmap of nqt + 1 bits
  if (tq > 1 && (int64_t)nqt + 1 > 524288)
    return fail(BSFA_ERR_UNSUPPORTED,
                "%d query tiles: more than 524287 with %d query heads per KV head", nqt, group);

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
  a.pattern = has_pattern(*mask) ? 1 : 0;
  a.dilation = mask->dilation;
  a.dil_span = mask->dilation_taps > 0
                   ? (int32_t)std::min<int64_t>((int64_t)mask->dilation * mask->dilation_taps,
                                                INT32_MAX)
                   : 0;
  a.block = mask->block;
  a.dil_bits = stride_pattern(mask->dilation);
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

int bsfa_decode_workspace_size(int32_t B, int32_t Hq, int32_t max_len, int32_t d,
                               int64_t* bytes) {
  if (!bytes) return fail(BSFA_ERR_INVALID_ARG, "bytes is required");
  if (B < 0 || Hq < 1 || max_len < 1)
    return fail(BSFA_ERR_INVALID_ARG, "need B >= 0, Hq >= 1, max_len >= 1");
  if (d != 64 && d != 128) return fail(BSFA_ERR_UNSUPPORTED, "head dim %d (need 64 or 128)", d);
  *bytes = (int64_t)B * Hq * decode_splits(max_len) * (d + 4) * (int64_t)sizeof(float);
  return ok();
}

}  // extern "C"

namespace {

// bsfa_decode and bsfa_decode_static. With fixed_scratch the per-split partials go to the
// library's fixed device scratch (workspace and workspace_bytes are ignored).
int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* lengths, void* out, float* lse, int32_t B, int32_t Hq,
                int32_t Hkv, int32_t max_len, int32_t d, const bsfa_strides* sq,
                const bsfa_strides* sk, const bsfa_strides* sv, const bsfa_strides* so,
                const bsfa_mask_spec* mask, const float* tau, float softmax_scale,
                int32_t out_dtype, uint64_t* stats, float* tile_max, uint8_t* keep,
                void* workspace, int64_t workspace_bytes, bool fixed_scratch, void* stream) {
  if (B < 0 || Hq < 1 || Hkv < 1 || max_len < 1)
    return fail(BSFA_ERR_INVALID_ARG, "need B >= 0, Hq >= 1, Hkv >= 1, max_len >= 1");
  if (Hq % Hkv != 0) return fail(BSFA_ERR_INVALID_ARG, "Hq (%d) %% Hkv (%d) != 0", Hq, Hkv);
  if (!mask) return fail(BSFA_ERR_INVALID_ARG, "mask is required");
  if (!valid_mask(mask))
    return fail(BSFA_ERR_INVALID_ARG,
                "mask fields must be >= 0 and random_ppm at most 1000000");
  if (out_dtype != BSFA_OUT_BF16 && out_dtype != BSFA_OUT_F32)
    return fail(BSFA_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale))
    return fail(BSFA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if ((tile_max == nullptr) != (keep == nullptr))
    return fail(BSFA_ERR_INVALID_ARG, "tile_max and keep must be given together");
  if (tile_max && !tau)
    return fail(BSFA_ERR_INVALID_ARG, "the per-block export needs tau (the gated path)");
  if (d != 64 && d != 128) return fail(BSFA_ERR_UNSUPPORTED, "head dim %d (need 64 or 128)", d);
  if (Hq / Hkv > 32)
    return fail(BSFA_ERR_UNSUPPORTED, "more than 32 query heads per KV head (%d)", Hq / Hkv);
  if (B == 0) return ok();
  if (!q || !k_cache || !v_cache || !lengths || !out || (!workspace && !fixed_scratch))
    return fail(BSFA_ERR_INVALID_ARG,
                "q, k_cache, v_cache, lengths, out and workspace are required");
  if (!sq || !sk || !sv || !so) return fail(BSFA_ERR_INVALID_ARG, "strides are required");
  if (!valid_strides(sq) || !valid_strides(sk) || !valid_strides(sv) || !valid_strides(so))
    return fail(BSFA_ERR_UNSUPPORTED, "strides must be non-negative multiples of 8 elements");
  if (!view_fits(sk, max_len, d) || !view_fits(sv, max_len, d))
    return fail(BSFA_ERR_UNSUPPORTED, "the K or V rows of one head span 2^31 bytes or more");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (!fixed_scratch && !aligned16(workspace)))
    return fail(BSFA_ERR_UNSUPPORTED,
                "q, k_cache, v_cache, out and workspace must be 16-byte aligned");
  if ((uintptr_t)lengths & 3u) return fail(BSFA_ERR_UNSUPPORTED, "lengths must be 4-byte aligned");
  const int32_t nsplit = decode_splits(max_len);
  const int64_t need = (int64_t)B * Hq * nsplit * (d + 4) * (int64_t)sizeof(float);
  if (fixed_scratch && need > bsfa::DEC_STATIC_SCRATCH_BYTES)
    return fail(BSFA_ERR_BUFFER_TOO_SMALL,
                "this decode step needs %lld bytes of scratch; the fixed scratch of "
                "bsfa_decode_static holds %lld (use bsfa_decode with a workspace)",
                (long long)need, (long long)bsfa::DEC_STATIC_SCRATCH_BYTES);
  if (!fixed_scratch && workspace_bytes < need)
    return fail(BSFA_ERR_BUFFER_TOO_SMALL, "workspace %lld bytes < %lld",
                (long long)workspace_bytes, (long long)need);
  // one dispatch counts its work-items in 32 bits
  if ((int64_t)B * Hkv * nsplit * bsfa::DEC_SPLIT_THREADS > (int64_t)UINT32_MAX ||
      (int64_t)B * Hq * (d / 32) * bsfa::DEC_COMBINE_THREADS > (int64_t)UINT32_MAX)
    return fail(BSFA_ERR_UNSUPPORTED, "grid too large");

  const char* err = nullptr;
  if (fixed_scratch) {
    const int rc = bsfa::decode_static_scratch(stream, &workspace, &err);
    if (rc != BSFA_OK) return fail(rc, "%s", err ? err : "fixed scratch unavailable");
  }

  bsfa::DecArgs a;
  memset(&a, 0, sizeof a);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.lengths = lengths;
  a.out = out;
  a.lse = lse;
  a.ws = (float*)workspace;
  a.sqb = sq->b; a.sqh = sq->h;
  a.skb = sk->b; a.skh = sk->h; a.skn = sk->n;
  a.svb = sv->b; a.svh = sv->h; a.svn = sv->n;
  a.sob = so->b; a.soh = so->h;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lmax = max_len;
  a.group = Hq / Hkv;
  a.nkb = (max_len + 63) / 64;
  a.nsplit = nsplit;
  a.causal = mask->causal != 0;
  a.window = mask->window;
  a.n_global = mask->n_global;
  a.pattern = has_pattern(*mask) ? 1 : 0;
  a.dilation = mask->dilation;
  a.block = mask->block;
  a.dil_span = mask->dilation_taps > 0
                   ? (int32_t)std::min<int64_t>((int64_t)mask->dilation * mask->dilation_taps,
                                                INT32_MAX)
                   : 0;
  a.random_ppm = mask->random_ppm;
  a.random_seed = mask->random_seed;
  a.force_diag = mask->force_keep_diag != 0;
  a.force_global = mask->force_keep_global != 0;
  a.dil_bits = stride_pattern(mask->dilation);
  a.tau = tau;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.stats = (unsigned long long*)stats;
  a.tile_max = tile_max;
  a.keep = keep;
  const int rc = bsfa::launch_decode(a, d, out_dtype == BSFA_OUT_F32, stream, &err);
  if (rc != BSFA_OK) return fail(rc, "%s", err ? err : "launch failed");
  return ok();
}

}  // namespace

extern "C" {

int bsfa_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* lengths, void* out, float* lse, int32_t B, int32_t Hq,
                int32_t Hkv, int32_t max_len, int32_t d, const bsfa_strides* sq,
                const bsfa_strides* sk, const bsfa_strides* sv, const bsfa_strides* so,
                const bsfa_mask_spec* mask, const float* tau, float softmax_scale,
                int32_t out_dtype, uint64_t* stats, float* tile_max, uint8_t* keep,
                void* workspace, int64_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, lengths, out, lse, B, Hq, Hkv, max_len, d, sq, sk,
                     sv, so, mask, tau, softmax_scale, out_dtype, stats, tile_max, keep,
                     workspace, workspace_bytes, false, stream);
}

int bsfa_decode_static(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* lengths, void* out, float* lse, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t max_len, int32_t d, const bsfa_strides* sq,
                       const bsfa_strides* sk, const bsfa_strides* sv,
                       const bsfa_strides* so, const bsfa_mask_spec* mask, const float* tau,
                       float softmax_scale, int32_t out_dtype, uint64_t* stats,
                       float* tile_max, uint8_t* keep, void* stream) {
  return decode_impl(q, k_cache, v_cache, lengths, out, lse, B, Hq, Hkv, max_len, d, sq, sk,
                     sv, so, mask, tau, softmax_scale, out_dtype, stats, tile_max, keep,
                     nullptr, 0, true, stream);
}

int bsfa_calibrate_workspace_size(int32_t Hq, int64_t* bytes) {
  if (!bytes) return fail(BSFA_ERR_INVALID_ARG, "bytes is required");
  if (Hq < 1) return fail(BSFA_ERR_INVALID_ARG, "need Hq >= 1");
  *bytes = calib_workspace_bytes(Hq);
  return ok();
}

int bsfa_calibrate_tau(const float* tile_max, const uint8_t* keep, int32_t B, int32_t Hq,
                       int64_t n_blocks, double quantile, float* tau, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (B < 0 || Hq < 1 || n_blocks < 0)
    return fail(BSFA_ERR_INVALID_ARG, "need B >= 0, Hq >= 1, n_blocks >= 0");
  if (!(quantile >= 0.0 && quantile <= 1.0))
    return fail(BSFA_ERR_INVALID_ARG, "quantile must lie in [0, 1]");
  if (!tau || !workspace) return fail(BSFA_ERR_INVALID_ARG, "tau and workspace are required");
  const int64_t per_head = (int64_t)B * n_blocks;
  if (per_head > 0 && (!tile_max || !keep))
    return fail(BSFA_ERR_INVALID_ARG, "tile_max and keep are required");
  if (per_head >= (int64_t)UINT32_MAX)
    return fail(BSFA_ERR_UNSUPPORTED, "2^32 - 1 or more blocks per head");
  const int64_t need = calib_workspace_bytes(Hq);
  if (workspace_bytes < need)
    return fail(BSFA_ERR_BUFFER_TOO_SMALL, "workspace %lld bytes < %lld",
                (long long)workspace_bytes, (long long)need);
  if (!aligned16(workspace) || ((uintptr_t)tile_max & 3u) || ((uintptr_t)tau & 3u))
    return fail(BSFA_ERR_UNSUPPORTED,
                "workspace must be 16-byte aligned, tile_max and tau 4-byte aligned");
  // one dispatch counts its work-items in 32 bits
  if (bsfa::calibrate_grid(B, Hq, n_blocks) * 256 > (int64_t)UINT32_MAX)
    return fail(BSFA_ERR_UNSUPPORTED, "grid too large");
  bsfa::CalibArgs a;
  memset(&a, 0, sizeof a);
  a.tile_max = tile_max;
  a.keep = keep;
  a.B = B;
  a.Hq = Hq;
  a.n_blocks = n_blocks;
  a.q = quantile;
  a.tau = tau;
  a.hist = reinterpret_cast<uint32_t*>(workspace);
  a.state = reinterpret_cast<bsfa::CalibState*>(reinterpret_cast<char*>(workspace) +
                                                (int64_t)Hq * 256 * sizeof(uint32_t));
  const char* err = nullptr;
  const int rc = bsfa::launch_calibrate(a, stream, &err);
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
  // no exception may cross the C ABI: a failed host allocation is an error code
  uint64_t* both = new (std::nothrow) uint64_t[2 * n];
  if (!both) return fail(BSFA_ERR_INVALID_ARG, "cannot allocate %zu host bytes", 2 * n * 8);
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
