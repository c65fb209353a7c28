// Block-sparse FlashAttention forward (prefill) for gfx950 (MI355X).
//
// Method: exact tiled attention with a running softmax ("sparse attention mechanism"
// glossary page, section "FlashAttention") plus the Block Sparse FlashAttention gate
// (AI Radio episode "Block Sparse Flash Attention", "The paper's summary" and "The
// paper's improvements"): for every (64-row query tile, 64-key block) the exact scores
// are computed first, their maximum is compared with a per-head threshold tau_h, and a
// block below it is dropped from the softmax and its V block is never loaded.
//
// Work decomposition
//   One workgroup of 512 threads serves four members that share one KV head, a member
//   being a (query head, 64-row query tile) pair: four heads of one query tile when the
//   group (query heads per KV head) is a multiple of four, two heads of two adjacent
//   query tiles when it is even, one head of four adjacent query tiles otherwise
//   (multi-head attention). Every staged K/V block thus feeds four 64-row query tiles.
//   The kernel is warp-specialised: per member, a producer wave owns all 64 rows (S^T,
//   gate, softmax, P to LDS) and a consumer wave accumulates O += P.V for them one step
//   behind; the consumers stage K and V.
//
// Register layout (v_mfma_f32_32x32x16_bf16; lane l, half h = l / 32, l32 = l % 32)
//   Scores are computed transposed, S^T = K Q^T (keys x queries), so a lane owns ONE
//   query row (l32) and 32 of its 64 keys: key = 32*mt + 8*(i/4) + 4*h + i%4 for
//   accumulator element i of key tile mt. The running max m and sum l are therefore
//   per-lane scalars; a row reduction is a local loop plus one exchange with lane l^32.
//   P^T is the B operand of the P.V MFMA (O^T = V^T P^T): for 16-key step ks the lane's
//   8 values are accumulator elements 8*(ks%2) .. +7 of tile ks/2; the producer writes
//   them to LDS in that operand layout for the consumer wave. V^T rows come from
//   a row-major V tile in LDS via ds_read_tr16_b64 (two 4-key reads per operand).
//
// The gate's tile maximum: local max over the lane's values, DPP all-reduce inside each
// 16-lane row, readlane across rows. The producer owns the whole tile and decides alone;
// the members' keep bytes meet in LDS at the step's barrier, so the V block is staged
// when any member keeps it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/bsfa.h"
#include "bsfa_internal.h"

namespace bsfa {
namespace {

#include "bsfa_device.h"

// The fields of the further primitives, read when a partial tile needs them. They are
// loaded from the kernel argument segment through an address the compiler cannot track,
// so the loads stay on this rare path instead of holding scalar registers for the whole
// kernel (the gated kernel has none to spare).
struct PatternArgs {
  int32_t pattern, dilation, block, dil_span;
  unsigned long long dil_bits;
};
__device__ __forceinline__ PatternArgs pattern_args() {
  auto base = (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(base));
  auto f = [&](size_t off) {
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(base + off);
  };
  PatternArgs p;
  p.pattern = f(offsetof(FwdArgs, pattern));
  p.dilation = f(offsetof(FwdArgs, dilation));
  p.block = f(offsetof(FwdArgs, block));
  p.dil_span = f(offsetof(FwdArgs, dil_span));
  p.dil_bits = *reinterpret_cast<const __attribute__((address_space(4))) unsigned long long*>(
      base + offsetof(FwdArgs, dil_bits));
  return p;
}

// Keys j0 + k, k in [0, 64), that query row i may attend, as bit k of the result: each
// static primitive (causal, N, window, dilated, blockwise, global tokens) is a range or
// a residue class of k; `rnd` says the random primitive selects this 64 x 64 tile.
__device__ __forceinline__ uint64_t row_mask(const FwdArgs& a, int i, int j0, bool rnd) {
  const PatternArgs pa = pattern_args();
  const int r = i - j0;  // k of the diagonal element (|r| < N < 2^31)
  uint64_t m = bits_below((int64_t)a.N - j0);
  if (a.causal) m &= bits_below((int64_t)r + 1);
  if (pa.pattern) {
    uint64_t p = (i < a.n_global) ? ~0ull : bits_below((int64_t)a.n_global - j0);
    if (a.window > 0)
      p |= bits_below((int64_t)r + a.window) & ~bits_below((int64_t)r - a.window + 1);
    if (pa.dilation > 0) {
      const int st = pa.dilation;
      const int off = ((r % st) + st) % st;  // keys k = off, off + st, ... below 64
      uint64_t dm = 0;
      if (off < 64) dm = (st >= 64 ? 1ull : pa.dil_bits) << off;
      if (pa.dil_span > 0)
        dm &= bits_below((int64_t)r + pa.dil_span) & ~bits_below((int64_t)r - pa.dil_span + 1);
      p |= dm;
    }
    if (pa.block > 0) {
      const int64_t lo = (int64_t)(i / pa.block) * pa.block;
      p |= bits_below(lo + pa.block - j0) & ~bits_below(lo - j0);
    }
    if (rnd) p = ~0ull;
    m &= p;
  }
  return i < a.N ? m : 0ull;
}


// Kernel modes: the dense path (no gate), the gated path, and the gated path that also
// exports every tile's maximum and keep bit (calibration and parity checks).
enum Mode { DENSE = 0, GATED = 1, GATED_EXPORT = 2 };

// Warp-specialised kernel. A workgroup serves four members that share one KV head, each
// member a (query head, 64-row query tile) pair: four heads of one query tile when the
// group has a multiple of four heads (TQ = 1), two heads of two adjacent query tiles
// (TQ = 2), or one head of four adjacent query tiles (TQ = 4, multi-head attention), so
// every staged K/V tile feeds four 64-row query tiles whatever the grouping. Per member,
// one producer wave owns the whole 64-row query tile: it computes S^T = K Q^T for both
// 32-row halves, takes the gate (the tile maximum is a wave reduction, with no exchange
// between waves), runs the softmax, and writes P in bf16 together with its rescale
// factors to LDS. One consumer wave of the same member accumulates O^T += V^T P^T for the
// 64 rows, one step behind. Waves h and h + 4 (producer and consumer of member h) share a
// SIMD, so the consumer's P.V MFMAs run beside the producer's softmax work. The consumers
// also stage every K and V tile (global loads into registers, then LDS), so the producers
// hold no staging registers.
// The workgroup steps through the union of its query tiles' key-block lists in ascending
// key-block order (a merge of the sorted lists, kept in scalar registers by every wave);
// a member whose own list lacks the step's block sits the step out (its scores are not
// used, and it neither keeps nor counts the block).
template <int D, int TQ, int MODE, bool OUT_F32>
__global__ __launch_bounds__(512) void bsfa_fwd_ws_kernel(const FwdArgs a) {
  constexpr int HPACK = 4;          // members per workgroup
  constexpr int HPK = HPACK / TQ;   // query heads per workgroup
  static_assert(TQ == 1 || TQ == 2 || TQ == 4, "members are 4 heads, 2 x 2 or 4 query tiles");
  constexpr bool GATE = MODE != DENSE;
  constexpr bool EXPORT = MODE == GATED_EXPORT;
  constexpr int NT = 256;  // threads that stage K/V tiles: the four consumer waves
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int KROW = D + 8;
  constexpr int VROW = D + 32;
  constexpr int NKF = 2 * KS;         // K fragments of one tile
  constexpr int EPF = 32 / KS;        // softmax elements per lane with each K fragment

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BLK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BLK * VROW];
  __shared__ bf16x8_t sP[2][HPACK][2][4][64];  // P^T operands: [buf][member][rh][ks][lane]
  __shared__ float sAlpha[2][HPACK][2][32];    // O rescale factor per row
  __shared__ uint32_t sFlag[2][HPACK];         // bit 0 keep, bits 1-2 rescale of rh 0/1
  __shared__ uint32_t sKeep[2];                // byte h: member h keeps the tile
  __shared__ float sL[HPACK][2][32];           // final row sums for the consumer
  __shared__ int sCount;                       // the workgroup's step count (TQ > 1)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const bool producer = wave < HPACK;
  const int h = wave & (HPACK - 1);  // member of the workgroup this wave serves
  const int mq = h % TQ;             // the member's query tile within the workgroup's

  // ---- which (batch, head pack, group of TQ query tiles) this workgroup owns.
  // Workgroups are dealt round-robin to the 8 XCDs. When the number of (batch, pack)
  // pairs is a multiple of 8, each XCD owns P / 8 consecutive packs and runs them one
  // after the other, so the workgroups resident on an XCD at a time mostly read one KV
  // head's K/V and share its L2. Query tile groups run longest-row first.
  const int packs = a.Hq / HPK;
  const int P = a.B * packs;
  const int ngrp = (a.nqt + TQ - 1) / TQ;
  const int wg = blockIdx.x;
  int p, trank;
  if (P % 8 == 0) {
    const int per = P / 8;
    const int l = wg / 8;  // the workgroup's place in its XCD's sequence
    p = (wg % 8) * per + l / ngrp;
    trank = l % ngrp;
  } else {
    p = wg % P;
    trank = wg / P;
  }
  const int b = p / packs, hp = p % packs;
  const int tg = (ngrp - 1 - trank) * TQ;  // first query tile of the workgroup
  const int t = tg + mq;                   // this member's query tile (>= nqt: no rows)
  const int hq = hp * HPK + h / TQ;
  const int g = (hp * HPK) / a.group;
  int qi[2];
  qi[0] = t * BLK + l32;
  qi[1] = t * BLK + 32 + l32;

  const int nkb = a.nqt;
  auto col_at = [&](int e) {
    const int c = ldc(a.col, e);
    return c < 0 ? 0 : (c > nkb ? nkb : c);
  };
  // Entry ranges [lo, hi) of the workgroup's query tiles. The per-list values live in
  // vectors, not arrays: an array indexed in a loop ends up in scratch or LDS.
  using ivec = int __attribute__((ext_vector_type(TQ == 1 ? 2 : TQ)));
  ivec lo, hi;
#pragma unroll
  for (int m = 0; m < TQ; ++m) {
    const int tm = tg + m;
    int e0 = 0, e1 = 0;
    if (tm < a.nqt) {
      e0 = ldc(a.row_ptr, tm);
      e1 = ldc(a.row_ptr, tm + 1);
      e0 = e0 < 0 ? 0 : (e0 > a.nnz ? (int)a.nnz : e0);
      e1 = e1 < e0 ? e0 : (e1 > a.nnz ? (int)a.nnz : e1);
    }
    lo[m] = e0;
    hi[m] = e1;
  }
  // Merge cursor over the TQ sorted lists: pos[m] is list m's next entry and cc[m] its key
  // block (kEnd once the list is exhausted); the union's next block is the least cc.
  constexpr int kEnd = 0x7FFFFFFF;
  struct Cursor {
    ivec pos, cc;
  };
  auto cur_init = [&](Cursor& u) {
#pragma unroll
    for (int m = 0; m < TQ; ++m) {
      u.pos[m] = lo[m];
      u.cc[m] = lo[m] < hi[m] ? col_at(lo[m]) : kEnd;
    }
  };
  auto cur_col = [&](const Cursor& u) {
    int c = u.cc[0];
#pragma unroll
    for (int m = 1; m < TQ; ++m) c = min(c, u.cc[m]);
    return c;  // kEnd: no steps left
  };
  auto cur_next = [&](Cursor& u) {
    const int c = cur_col(u);
#pragma unroll
    for (int m = 0; m < TQ; ++m)
      if (u.cc[m] == c) {
        ++u.pos[m];
        u.cc[m] = u.pos[m] < hi[m] ? col_at(u.pos[m]) : kEnd;
      }
  };

  const uint32_t k_bytes = (uint32_t)(((int64_t)(a.N - 1) * a.skn + D) * 2);
  const uint32_t v_bytes = (uint32_t)(((int64_t)(a.N - 1) * a.svn + D) * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + (int64_t)b * a.skb + (int64_t)g * a.skh), (short)0, (int)k_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v + (int64_t)b * a.svb + (int64_t)g * a.svh), (short)0, (int)v_bytes, 0x00020000);
  const uint32_t k_tile_bytes = (uint32_t)(BLK * a.skn * 2);
  const uint32_t v_tile_bytes = (uint32_t)(BLK * a.svn * 2);
  using ST = Stage<D, NT>;

  Cursor first;
  cur_init(first);
  const int c_first = cur_col(first);  // kEnd: the workgroup has no steps

  // ---- the number of steps: the size of the union of the members' lists. With one
  // query tile that is its list's length. With several, the workgroup marks the key
  // blocks of its tiles' entries (one contiguous run of the lists) in an LDS bitmap,
  // borrowed from the P buffers before their first use, and counts the marks.
  int nsteps;
  if constexpr (TQ == 1) {
    nsteps = hi[0] - lo[0];
  } else {
    uint32_t* bits = reinterpret_cast<uint32_t*>(&sP[0][0][0][0][0]);
    const int nwords = (nkb + 1 + 31) >> 5;  // key blocks 0 .. nkb (col_at's clamp)
    int e_hi = hi[0];
#pragma unroll
    for (int m = 1; m < TQ; ++m) e_hi = max(e_hi, hi[m]);
    for (int w = tid; w < nwords; w += 512) bits[w] = 0u;
    if (tid == 0) sCount = 0;
    __syncthreads();
    for (int e = lo[0] + tid; e < e_hi; e += 512) {
      int cb = a.col[e];
      cb = cb < 0 ? 0 : (cb > nkb ? nkb : cb);
      atomicOr(&bits[cb >> 5], 1u << (cb & 31));
    }
    __syncthreads();
    int cnt = 0;
    for (int w = tid; w < nwords; w += 512) cnt += __builtin_popcount(bits[w]);
    if (cnt) atomicAdd(&sCount, cnt);
    __syncthreads();
    nsteps = __builtin_amdgcn_readfirstlane(sCount);
    __syncthreads();  // the P buffers are free again
  }

  // Whether some member keeps the step in keep slot s (read by the consumers after the
  // step's barrier): the V tile is staged only then.
  auto any_of = [&](int s) -> bool {
    if constexpr (GATE) return sKeep[s] != 0u;
    return true;
  };

  if (producer) {
    // ================================ producer ================================
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const uint16_t* qrow =
          a.q + (int64_t)b * a.sqb + (int64_t)hq * a.sqh + (int64_t)qi[rh] * a.sqn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[rh][ks] = qi[rh] < a.N
                         ? *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16 + half * 8)
                         : bf16x8_t{};
    }
    const float tau = GATE ? ldc(a.tau, hq) : 0.0f;
    const int kbase_el = l32 * KROW + half * 8;
    auto k_frag = [&](const uint16_t* tile, int f) {
      const int mt = f & 1, ks = f >> 1;
      return *reinterpret_cast<const bf16x8_t*>(tile + kbase_el + mt * 32 * KROW + ks * 16);
    };
    auto mask_max = [&](f32x16_t (&s)[2][2], int c, int cls, float (&mx)[2]) {
      if (cls & BSFA_CLS_PARTIAL) {
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const uint64_t m = row_mask(a, qi[rh], c * BLK, (cls & BSFA_CLS_RANDOM) != 0);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const uint32_t w = (uint32_t)(m >> (32 * mt)) >> (4 * half);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              // A select, not an and/or blend of the bits: this compiler lowers the blend
              // to v_bitop3_b32 forms that gave wrong elements.
              const uint32_t bit = __builtin_amdgcn_ubfe(w, 8 * (i >> 2) + (i & 3), 1);
              s[rh][mt][i] = bit ? s[rh][mt][i] : -INFINITY;
            }
          }
        }
      }
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) m = fmaxf(m, s[rh][mt][i]);
        mx[rh] = m;
      }
    };
    struct PState {
      float mx[2];
      float tmax;
      bool keep;
      bool in;  // the member's own list has this step's block
      int e;    // the member's entry of this step's block (when in)
    };
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.0f, 0.0f};
    unsigned n_kept = 0, n_skip = 0;
    const float c2 = a.scale_log2;
    auto gate = [&](PState& st, int cls, int slot) {
      if constexpr (GATE) {
        const float tm = wave_max(fmaxf(st.mx[0], st.mx[1])) * a.scale;
        st.tmax = tm;
        st.keep = st.in && ((cls & BSFA_CLS_FORCED) != 0 || tm >= tau);
        if (lane == 0) reinterpret_cast<volatile uint8_t*>(&sKeep[slot])[h] = st.keep ? 1 : 0;
      } else {
        st.keep = st.in;
      }
    };
    // Running reference max of each row (raw units), raised lazily: only when some row of
    // the 32-row half grows past it by more than 2 in exp2 units (or gets its first keys),
    // so P <= 4 and O rarely needs rescaling (2.7 % of row-half steps at the 64K sink/local
    // shape). A larger margin rescales less, but then a row's dominant P is an arbitrary
    // bf16-rounded value up to 2^margin instead of about 1: with 8 (P <= 256), rows whose
    // weight sits on a few keys erred by up to 1.1e-2 in O.
    auto softmax_prep = [&](int rh, float mx, bool& rescale, float& alpha) -> float {
      float x0, x1;
      pair32(mx, x0, x1);
      const float m_new = fmaxf(m_run[rh], fmaxf(x0, x1));
      const bool grow =
          (m_run[rh] == -INFINITY) ? (m_new != -INFINITY) : ((m_new - m_run[rh]) * c2 > 2.0f);
      rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
      alpha = 1.0f;
      if (rescale) {
        alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f((m_run[rh] - m_new) * c2);
        m_run[rh] = m_new;
        l_run[rh] *= alpha;
      }
      return (m_run[rh] == -INFINITY ? 0.0f : m_run[rh]) * c2;
    };
    // Softmax of a kept tile: the P^T operands to LDS, the row sums, the flags.
    auto publish_prep = [&](const PState& cur, int buf, float (&mb)[2]) {
      bool resc[2];
      float alpha[2];
      mb[0] = softmax_prep(0, cur.mx[0], resc[0], alpha[0]);
      mb[1] = softmax_prep(1, cur.mx[1], resc[1], alpha[1]);
      if (half == 0) {
        if (resc[0]) sAlpha[buf][h][0][l32] = alpha[0];
        if (resc[1]) sAlpha[buf][h][1][l32] = alpha[1];
      }
      if (lane == 0) sFlag[buf][h] = 1u | (resc[0] ? 2u : 0u) | (resc[1] ? 4u : 0u);
    };
    auto count_export = [&](const PState& st) {
      if (!st.in) return;
      if (st.keep) ++n_kept; else ++n_skip;
      if (EXPORT && lane == 0) {
        const int64_t idx = ((int64_t)b * a.Hq + hq) * a.nnz + st.e;
        a.tile_max[idx] = st.tmax;
        a.keep[idx] = st.keep ? 1 : 0;
      }
    };

    f32x16_t sA[2][2], sB[2][2];
    PState stA{{-INFINITY, -INFINITY}, 0.0f, false, false, 0};
    PState stB{{-INFINITY, -INFINITY}, 0.0f, false, false, 0};
    Cursor nx = first;  // the next block to score
    // The member's part in the step at the cursor; moves the cursor on.
    auto take = [&](PState& st) -> int2 {
      const int c = cur_col(nx);
      // the member's list, selected by unrolled compares: indexing the cursor arrays by
      // the (wave-uniform) member would put them in scratch or LDS
      int my_c = nx.cc[0], my_e = nx.pos[0];
#pragma unroll
      for (int m = 1; m < TQ; ++m)
        if (m == mq) {
          my_c = nx.cc[m];
          my_e = nx.pos[m];
        }
      st.in = TQ == 1 || my_c == c;
      st.e = my_e;
      const int cls = st.in ? ldc_byte(a.cls, st.e) : 0;
      cur_next(nx);
      return make_int2(c, cls);
    };

    // Step i: the softmax of step i's tile (scores sc, state cur) interleaved with the
    // scores of step i + 1 (into sn, state nxt).
    auto pstep = [&](auto keep_tag, const int i, f32x16_t (&sc)[2][2], PState& cur,
                     f32x16_t (&sn)[2][2], PState& nxt) {
      constexpr bool KEEP = decltype(keep_tag)::value;
      const int buf = i & 1;
      const uint16_t* kt = sK[(i + 1) & 1];
      float mb[2] = {0.0f, 0.0f};
      if constexpr (KEEP) publish_prep(cur, buf, mb);
      else if (lane == 0) sFlag[buf][h] = 0u;
      float rs[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sn[rh][mt] = f32x16_t{};
      // K fragments read ahead. A skipped step (QK^T and the maximum only) reads 4 ahead
      // and pins each read in place: left free, the scheduler moved the reads next to
      // their MFMAs and waited out every read's latency.
      constexpr int PF = KEEP ? 2 : 4;
      bf16x8_t kf[PF];
      auto fr = [](int n) { return 2 * (n % KS) + n / KS; };  // key half outer
#pragma unroll
      for (int n = 0; n < PF; ++n) kf[n] = k_frag(kt, fr(n));
      bf16x8_t pb[2][2];  // the chunks of the current key half, [rh][ks2 % 2]
#pragma unroll
      for (int n = 0; n < NKF; ++n) {
        const bf16x8_t kcur = kf[n % PF];
        if (n + PF < NKF) kf[n % PF] = k_frag(kt, fr(n + PF));
        if constexpr (!KEEP) __builtin_amdgcn_sched_barrier(0);
        const int f = fr(n), mt = f & 1, ks = f >> 1;
        sn[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[0][ks], sn[0][mt], 0, 0, 0);
        sn[1][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[1][ks], sn[1][mt], 0, 0, 0);
        if constexpr (KEEP) {
#pragma unroll
          for (int u = 0; u < EPF; ++u) {
            const int j = (n % KS) * EPF + u;  // element j of this key half
            const int rh = j >> 4, el = j & 15, mh = n / KS;
            const float pv_ = __builtin_amdgcn_exp2f(fmaf(sc[rh][mh][el], c2, -mb[rh]));
            rs[rh][j & 1] += pv_;
            pb[rh][el >> 3][el & 7] = (__bf16)pv_;
            if ((el & 7) == 7)  // a chunk of 8 is complete: P^T operand of step 2*mh + el/8
              sP[buf][h][rh][2 * mh + (el >> 3)][lane] = pb[rh][el >> 3];
          }
        }
      }
      if constexpr (KEEP) {
        l_run[0] += rs[0][0] + rs[0][1];
        l_run[1] += rs[1][0] + rs[1][1];
      }
      const int2 cn = take(nxt);
      mask_max(sn, cn.x, cn.y, nxt.mx);
      gate(nxt, cn.y, (i + 1) & 1);
      __syncthreads();  // P(i), V(i), K(i+2) and the keep bytes of step i+1 are visible
      count_export(cur);
    };

    if (c_first != kEnd) {
      const int2 c0 = take(stA);
      __syncthreads();  // (1) K of steps 0 and 1 staged by the consumers
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sA[rh][mt] = f32x16_t{};
#pragma unroll
      for (int f = 0; f < NKF; ++f) {
        const bf16x8_t kcur = k_frag(sK[0], f);
        const int mt = f & 1, ks = f >> 1;
        sA[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[0][ks], sA[0][mt], 0, 0, 0);
        sA[1][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[1][ks], sA[1][mt], 0, 0, 0);
      }
      mask_max(sA, c0.x, c0.y, stA.mx);
      gate(stA, c0.y, 0);
      __syncthreads();  // (2) keep bytes of step 0; every wave is done reading sK[0]

      // Unrolled by two so the scores alternate between sA and sB without copies. The
      // loop has no exit between its two steps, and its bound is the step count: other
      // forms of the same control flow (an exit between the steps, a bound read from the
      // cursors) cost this compiler registers it does not have.
      int i = 0;
      for (; i + 2 < nsteps; i += 2) {  // steps i + 1 and i + 2 exist
        if (stA.keep) pstep(std::true_type{}, i, sA, stA, sB, stB);
        else pstep(std::false_type{}, i, sA, stA, sB, stB);
        if (stB.keep) pstep(std::true_type{}, i + 1, sB, stB, sA, stA);
        else pstep(std::false_type{}, i + 1, sB, stB, sA, stA);
      }
      if (i + 1 < nsteps) {
        if (stA.keep) pstep(std::true_type{}, i, sA, stA, sB, stB);
        else pstep(std::false_type{}, i, sA, stA, sB, stB);
#pragma unroll
        for (int rh = 0; rh < 2; ++rh)
#pragma unroll
          for (int m = 0; m < 2; ++m) sA[rh][m] = sB[rh][m];
        stA = stB;
        ++i;
      }
      // the last step: its softmax, then V(last) staged
      const int buf = i & 1;
      if (stA.keep) {
        float mb[2];
        publish_prep(stA, buf, mb);
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          float rs = 0.0f;
#pragma unroll
          for (int ks2 = 0; ks2 < 4; ++ks2) {
            bf16x8_t pb;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int j = 8 * ks2 + u;
              const float pv_ =
                  __builtin_amdgcn_exp2f(fmaf(sA[rh][j >> 4][j & 15], c2, -mb[rh]));
              rs += pv_;
              pb[u] = (__bf16)pv_;
            }
            sP[buf][h][rh][ks2][lane] = pb;
          }
          l_run[rh] += rs;
        }
      } else if (lane == 0) {
        sFlag[buf][h] = 0u;
      }
      // final row sums for the consumer; the producer writes LSE
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        float l0, l1;
        pair32(l_run[rh], l0, l1);
        const float l_tot = l0 + l1;
        if (half == 0) sL[h][rh][l32] = l_tot;
        if (a.lse && half == 0 && qi[rh] < a.N)
          a.lse[((int64_t)b * a.Hq + hq) * a.N + qi[rh]] =
              l_tot > 0.0f ? m_run[rh] * a.scale + logf(l_tot) : -INFINITY;
      }
      __syncthreads();  // (last) P(last), V(last), row sums visible
      count_export(stA);
    } else {
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
        if (a.lse && half == 0 && qi[rh] < a.N)
          a.lse[((int64_t)b * a.Hq + hq) * a.N + qi[rh]] = -INFINITY;
    }
    if (a.stats && lane == 0) {
      unsigned long long* st = a.stats + ((int64_t)b * a.Hq + hq) * 2;
      atomicAdd(st, (unsigned long long)n_kept);
      atomicAdd(st + 1, (unsigned long long)n_skip);
    }
  } else {
    // ================================ consumer ================================
    const int ctid = tid - 64 * HPACK;  // 0 .. 255
    ST stk, stv;
    stk.init(ctid, a.skn);
    stv.init(ctid, a.svn);
    u32x4_t kr[ST::CPT], vr[ST::CPT];
    const int jl = lane & 15;
    const int vbase_el = (4 * half + (jl >> 2)) * VROW + 16 * ((lane >> 4) & 1) + 4 * (jl & 3);
    f32x16_t o[2][DT];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rh][dt] = f32x16_t{};

    // O^T += V(slot)^T P(slot)^T for the tile whose flags sit in sFlag[slot][h].
    auto pv = [&](int slot) {
      const uint32_t fl = sFlag[slot][h];
      if ((fl & 1u) == 0u) return;
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        if (fl & (2u << rh)) {
          const float alpha = sAlpha[slot][h][rh][l32];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rh][dt][r] *= alpha;
        }
      }
      const uint16_t* vt = sV[slot] + vbase_el;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t p0 = sP[slot][h][0][ks][lane];
        const bf16x8_t p1 = sP[slot][h][1][ks][lane];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* q0 = vt + 16 * ks * VROW + 32 * dt;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(q0));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(q0 + 8 * VROW));
          // Whole-vector concatenation and bit cast: an element-by-element copy from the
          // two i16x4 results into a bf16x8 is lowered with a wrong v_perm_b32 (it
          // duplicated element 0) by this compiler.
          const i16x8_t cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, cat);
          o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p0, o[0][dt], 0, 0, 0);
          o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1, o[1][dt], 0, 0, 0);
        }
      }
    };

    if (c_first != kEnd) {
      // The K stream runs two steps ahead of the V stream.
      Cursor kc = first, vc = first;
      // prologue, in step with the producers' barriers (1) and (2)
      stk.load(kr, krs, (uint32_t)c_first * k_tile_bytes);
      cur_next(kc);
      ST::template store<KROW>(sK[0], kr, ctid);
      int ck = cur_col(kc);
      if (ck != kEnd) {
        stk.load(kr, krs, (uint32_t)ck * k_tile_bytes);
        cur_next(kc);
        ST::template store<KROW>(sK[1], kr, ctid);
      }
      __syncthreads();  // (1)
      __syncthreads();  // (2)
      bool any_cur = any_of(0);
      if (any_cur) stv.load(vr, vrs, (uint32_t)c_first * v_tile_bytes);
      cur_next(vc);
      ck = cur_col(kc);
      bool k_pending = ck != kEnd;  // K of step i + 2 is in registers
      if (k_pending) {
        stk.load(kr, krs, (uint32_t)ck * k_tile_bytes);
        cur_next(kc);
      }
      int i = 0;
      for (; cur_col(vc) != kEnd; ++i) {  // step i + 1 exists
        const int buf = i & 1;
        if (i > 0) pv((i - 1) & 1);  // P.V of the step before
        if (any_cur) ST::template store<VROW>(sV[buf], vr, ctid);
        if (k_pending) ST::template store<KROW>(sK[buf], kr, ctid);
        __syncthreads();
        ck = cur_col(kc);
        k_pending = ck != kEnd;
        if (k_pending) {
          stk.load(kr, krs, (uint32_t)ck * k_tile_bytes);
          cur_next(kc);
        }
        const int c_n = cur_col(vc);
        cur_next(vc);
        any_cur = any_of((i + 1) & 1);
        if (any_cur) stv.load(vr, vrs, (uint32_t)c_n * v_tile_bytes);
      }
      {
        const int buf = i & 1;
        if (i > 0) pv((i - 1) & 1);
        if (any_cur) ST::template store<VROW>(sV[buf], vr, ctid);
        __syncthreads();  // (last)
        pv(buf);
      }
    }

    // ---- epilogue: O = O^T / l, one store per element
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const int q = qi[rh];
      if (q >= a.N) continue;
      const float l_tot = c_first != kEnd ? sL[h][rh][l32] : 0.0f;
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const int64_t obase = (int64_t)b * a.sob + (int64_t)hq * a.soh + (int64_t)q * a.son;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = 32 * dt + 8 * r + 4 * half;
          const f32x16_t& oo = o[rh][dt];
          if constexpr (OUT_F32) {
            float* op = reinterpret_cast<float*>(a.out) + obase + d0;
            *reinterpret_cast<float4*>(op) = make_float4(oo[4 * r] * inv, oo[4 * r + 1] * inv,
                                                         oo[4 * r + 2] * inv, oo[4 * r + 3] * inv);
          } else {
            uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + obase + d0;
            u32x2_t w;
            const __bf16 v0 = (__bf16)(oo[4 * r] * inv), v1 = (__bf16)(oo[4 * r + 1] * inv);
            const __bf16 v2 = (__bf16)(oo[4 * r + 2] * inv), v3 = (__bf16)(oo[4 * r + 3] * inv);
            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
            *reinterpret_cast<u32x2_t*>(op) = w;
          }
        }
    }
  }
}

template <int D, int TQ, int MODE, bool OUT_F32>
hipError_t launch_ws_variant(const FwdArgs& a, hipStream_t stream) {
  const int64_t groups = (a.nqt + TQ - 1) / TQ;
  const unsigned grid = (unsigned)((int64_t)a.B * (a.Hq / (4 / TQ)) * groups);
  hipLaunchKernelGGL((bsfa_fwd_ws_kernel<D, TQ, MODE, OUT_F32>), dim3(grid), dim3(512), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int TQ>
hipError_t launch_ws(const FwdArgs& a, bool out_f32, hipStream_t s) {
  if (a.tau == nullptr)
    return out_f32 ? launch_ws_variant<D, TQ, DENSE, true>(a, s)
                   : launch_ws_variant<D, TQ, DENSE, false>(a, s);
  if (a.tile_max != nullptr)
    return out_f32 ? launch_ws_variant<D, TQ, GATED_EXPORT, true>(a, s)
                   : launch_ws_variant<D, TQ, GATED_EXPORT, false>(a, s);
  return out_f32 ? launch_ws_variant<D, TQ, GATED, true>(a, s)
                 : launch_ws_variant<D, TQ, GATED, false>(a, s);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int hpack, bool out_f32, hipStream_t s) {
  switch (hpack) {
    case 4: return launch_ws<D, 1>(a, out_f32, s);
    case 2: return launch_ws<D, 2>(a, out_f32, s);
    default: return launch_ws<D, 4>(a, out_f32, s);
  }
}

}  // namespace

int launch_fwd(const FwdArgs& a, int d, int hpack, bool out_f32, void* stream, const char** err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = d == 64 ? launch_d<64>(a, hpack, out_f32, s) : launch_d<128>(a, hpack, out_f32, s);
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return BSFA_ERR_HIP;
  }
  return BSFA_OK;
}

int copy_to_host_sync(void* dst, const void* src, size_t bytes, void* stream, const char** err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return BSFA_ERR_HIP;
  }
  return BSFA_OK;
}

}  // namespace bsfa
