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
//   One workgroup = one 64-row query tile of HPACK query heads that share a KV head
//   (grouped-query attention), so each staged K/V block feeds HPACK heads; 128 * HPACK
//   threads. Two kernels:
//   - packs of four heads (bsfa_fwd_ws_kernel): warp-specialised. Per head, a producer
//     wave owns all 64 rows (S^T, gate, softmax, P to LDS) and a consumer wave
//     accumulates O += P.V for them one step behind; the consumers stage K and V.
//   - packs of one or two heads (bsfa_fwd_kernel): lock-step, two waves per head with
//     32 query rows each, every wave running every phase.
//
// Register layout (v_mfma_f32_32x32x16_bf16; lane l, half h = l / 32, l32 = l % 32)
//   Scores are computed transposed, S^T = K Q^T (keys x queries), so a lane owns ONE
//   query row (l32) and 32 of its 64 keys: key = 32*mt + 8*(i/4) + 4*h + i%4 for
//   accumulator element i of key tile mt. The running max m and sum l are therefore
//   per-lane scalars; a row reduction is a local loop plus one exchange with lane l^32.
//   P^T is the B operand of the P.V MFMA (O^T = V^T P^T): for 16-key step ks the lane's
//   8 values are accumulator elements 8*(ks%2) .. +7 of tile ks/2. The lock-step kernel
//   feeds them straight from the accumulator registers; the warp-specialised kernel
//   writes them to LDS in that operand layout for the consumer wave. V^T rows come from
//   a row-major V tile in LDS via ds_read_tr16_b64 (two 4-key reads per operand).
//
// The gate's tile maximum: local max over the lane's values, DPP all-reduce inside each
// 16-lane row, readlane across rows. In the lock-step kernel it then goes through one LDS
// slot per wave and a barrier, so the keep/skip branch is uniform across the workgroup;
// in the warp-specialised kernel the producer owns the whole tile and decides alone.
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

struct TileState {
  float mx;    // this lane's maximum of the tile's raw scores
  float tmax;  // the head's block maximum in scaled units (gated modes)
  bool keep;   // this head keeps the tile
  bool any;    // some head of the workgroup keeps it (its V block is loaded)
};

// Software pipeline over the query tile's block list, one barrier per tile. Step e:
//   S(e+1) = K(e+1) Q^T interleaved with P(e) = exp(S(e) - m)   (K(e+1) already staged)
//   block max of S(e+1) -> LDS; V(e) and K(e+2) registers -> LDS
//   barrier
//   gate(e+1)
//   O += P(e) V(e)
//   issue loads of V(e+1) (only if some head keeps e+1) and K(e+3)
// so each load's latency is covered by the next step's QK^T/softmax block, and the
// staging registers are free while P.V runs.
template <int D, int HPACK, int MODE, bool OUT_F32>
__global__ __launch_bounds__(128 * HPACK) void bsfa_fwd_kernel(const FwdArgs a) {
  constexpr bool GATE = MODE != DENSE;
  constexpr bool EXPORT = MODE == GATED_EXPORT;
  constexpr int NW = 2 * HPACK;  // waves per workgroup
  constexpr int NT = 64 * NW;
  constexpr int KS = D / 16;     // 16-wide steps along d for S^T = K Q^T
  constexpr int DT = D / 32;     // 32-row tiles of O^T along d
  constexpr int KROW = D + 8;    // K tile row stride (elements)
  constexpr int VROW = D + 32;   // V tile row stride (elements)
  constexpr int NQK = 2 * KS;    // MFMAs in one QK^T tile
  constexpr int EPS = 32 / NQK;  // softmax elements per lane interleaved with each MFMA

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BLK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BLK * VROW];
  __shared__ float sRed[2][NW];

  const int tid = threadIdx.x;
  // wave index as a wave-uniform (scalar) value, so per-wave quantities stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- which (batch, head pack, query tile) this workgroup owns.
  // Workgroups are dealt round-robin to the 8 XCDs; when the number of (batch, pack)
  // pairs is a multiple of 8, consecutive packs (same KV head) land on the same XCD,
  // so its L2 serves one KV head's K/V. Query tiles run longest-row first.
  const int packs = a.Hq / HPACK;
  const int P = a.B * packs;
  const int wg = blockIdx.x;
  int p, trank;
  if (P % 8 == 0) {
    const int per = P / 8;
    p = (wg % 8) * per + (wg / 8) % per;
    trank = wg / P;
  } else {
    p = wg % P;
    trank = wg / P;
  }
  const int b = p / packs, hp = p % packs;
  const int t = a.nqt - 1 - trank;
  const int hq = hp * HPACK + (wave >> 1);
  const int g = (hp * HPACK) / a.group;  // every head of the pack shares this KV head
  const int qi = t * BLK + (wave & 1) * 32 + l32;  // this lane's query row

  // ---- Q^T fragments (B operand of S^T = K Q^T): d = 16*ks + 8*half + [0, 8)
  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = a.q + (int64_t)b * a.sqb + (int64_t)hq * a.sqh + (int64_t)qi * a.sqn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qi < a.N)
        qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16 + half * 8);
      else
        qf[ks] = bf16x8_t{};
    }
  }

  float tau_pack[HPACK];
#pragma unroll
  for (int j = 0; j < HPACK; ++j) tau_pack[j] = GATE ? ldc(a.tau, hp * HPACK + j) : 0.0f;

  int e0 = ldc(a.row_ptr, t), e1 = ldc(a.row_ptr, t + 1);
  e0 = e0 < 0 ? 0 : (e0 > a.nnz ? (int)a.nnz : e0);
  e1 = e1 < e0 ? e0 : (e1 > a.nnz ? (int)a.nnz : e1);
  const int nkb = a.nqt;  // key blocks = query tiles (square 64x64 tiles)
  auto col_at = [&](int e) {
    const int c = ldc(a.col, e);
    return c < 0 ? 0 : (c > nkb ? nkb : c);
  };

  // Buffer views of this (batch, KV head)'s K and V rows: exactly N rows.
  const uint32_t k_bytes = (uint32_t)(((int64_t)(a.N - 1) * a.skn + D) * 2);
  const uint32_t v_bytes = (uint32_t)(((int64_t)(a.N - 1) * a.svn + D) * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + (int64_t)b * a.skb + (int64_t)g * a.skh), (short)0, (int)k_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v + (int64_t)b * a.svb + (int64_t)g * a.svh), (short)0, (int)v_bytes, 0x00020000);
  const uint32_t k_tile_bytes = (uint32_t)(BLK * a.skn * 2);
  const uint32_t v_tile_bytes = (uint32_t)(BLK * a.svn * 2);
  using ST = Stage<D, NT>;
  ST stk, stv;
  stk.init(tid, a.skn);
  stv.init(tid, a.svn);

  // LDS read bases: K operand rows (l32 [+32]) at d = 16*ks + 8*half; V^T transpose
  // reads at row 4*half + jl/4, column 16*((lane/16)%2) + 4*(jl%4) of each 16-key step.
  const int kbase_el = l32 * KROW + half * 8;
  const int jl = lane & 15;
  const int vbase_el = (4 * half + (jl >> 2)) * VROW + 16 * ((lane >> 4) & 1) + 4 * (jl & 3);

  // K fragment (A operand) of S^T MFMA step st: key tile mt = st % 2, d-step ks = st / 2.
  auto k_frag = [&](const uint16_t* tile, int st) {
    const int mt = st & 1, ks = st >> 1;
    return *reinterpret_cast<const bf16x8_t*>(tile + kbase_el + mt * 32 * KROW + ks * 16);
  };
  // One S^T MFMA step st of QK^T (the two accumulator chains alternate).
  auto qk_step = [&](const uint16_t* tile, f32x16_t (&s)[2], int st) {
    s[st & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(tile, st), qf[st >> 1],
                                                        s[st & 1], 0, 0, 0);
  };

  // Mask a PARTIAL tile element-wise and return this lane's maximum (raw units).
  auto mask_max = [&](f32x16_t (&s)[2], int c, int cls) -> float {
    if (cls & BSFA_CLS_PARTIAL) {
      // Element i of chain mt holds key mt*32 + 8*(i/4) + 4*half + i%4 of the block.
      const uint64_t m = row_mask(a, qi, c * BLK, (cls & BSFA_CLS_RANDOM) != 0);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint32_t w = (uint32_t)(m >> (32 * mt)) >> (4 * half);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // A select, not an and/or blend of the bits: this compiler lowers the blend to
          // v_bitop3_b32 forms that gave wrong elements.
          const uint32_t bit = __builtin_amdgcn_ubfe(w, 8 * (i >> 2) + (i & 3), 1);
          s[mt][i] = bit ? s[mt][i] : -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mt][i]);
    return mx;
  };

  // Per-head keep decisions for the tile whose wave maxima sit in sRed[slot].
  auto decide = [&](int slot, int cls, TileState& st) {
    const bool forced = (cls & BSFA_CLS_FORCED) != 0;
    st.any = false;
#pragma unroll
    for (int j = 0; j < HPACK; ++j) {
      const float tm = fmaxf(sRed[slot][2 * j], sRed[slot][2 * j + 1]) * a.scale;
      const bool kj = forced || (tm >= tau_pack[j]);
      if (j == (wave >> 1)) {
        st.keep = kj;
        st.tmax = tm;
      }
      st.any = st.any || kj;
    }
  };

  float m_run = -INFINITY;  // reference max (raw q.k units) of this lane's row
  float l_run = 0.0f;       // this lane's share of sum exp(scale * (s - m_run))
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};
  unsigned n_kept = 0, n_skip = 0;
  const float c2 = a.scale_log2;

  u32x4_t kr[Stage<D, NT>::CPT], vr[Stage<D, NT>::CPT];
  f32x16_t sA[2], sB[2];
  TileState stA{-INFINITY, 0.0f, false, false}, stB{-INFINITY, 0.0f, false, false};

  // Softmax bookkeeping for a kept tile: the reference max is raised only when some
  // row's max grows by more than 2^8 in exp2 units (or on a row's first keys), so
  // P <= 256 and O rarely needs rescaling. Returns the exp2 offset for the tile.
  auto softmax_prep = [&](float mx, bool& rescale, float& alpha) -> float {
    float x0, x1;
    pair32(mx, x0, x1);
    const float m_new = fmaxf(m_run, fmaxf(x0, x1));
    const bool grow =
        (m_run == -INFINITY) ? (m_new != -INFINITY) : ((m_new - m_run) * c2 > 8.0f);
    rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
    alpha = 1.0f;
    if (rescale) {
      alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      m_run = m_new;
      l_run *= alpha;
    }
    return (m_run == -INFINITY ? 0.0f : m_run) * c2;
  };

  // O^T += V(tile)^T P^T, after applying a pending rescale.
  auto pv = [&](const uint16_t* vtile, const bf16x8_t (&pb)[4], bool rescale, float alpha) {
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const uint16_t* vt = vtile + vbase_el;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* p0 = vt + 16 * ks * VROW + 32 * dt;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(p0));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(p0 + 8 * VROW));
        // Whole-vector concatenation and bit cast: an element-by-element copy from the
        // two i16x4 results into a bf16x8 is lowered with a wrong v_perm_b32 (it
        // duplicated element 0) by this compiler.
        const i16x8_t cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, cat);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[dt], 0, 0, 0);
      }
    }
  };

  auto count_export = [&](int e, const TileState& st) {
    if (st.keep) ++n_kept; else ++n_skip;
    if (EXPORT && (wave & 1) == 0 && lane == 0) {
      const int64_t idx = ((int64_t)b * a.Hq + hq) * a.nnz + e;
      a.tile_max[idx] = st.tmax;
      a.keep[idx] = st.keep ? 1 : 0;
    }
  };

  // One pipeline step for tile e (scores in sc, state cur) that also produces tile e+1
  // (sn, nxt); e + 1 < e1. KEEP is cur.keep, so each variant is straight-line code.
  auto step = [&](auto keep_tag, const int e, f32x16_t (&sc)[2], TileState& cur,
                  f32x16_t (&sn)[2], TileState& nxt) {
    constexpr bool KEEP = decltype(keep_tag)::value;
    const int i = e - e0;
    const uint16_t* kt_next = sK[(i + 1) & 1];
    bool rescale = false;
    float alpha = 1.0f, mb = 0.0f;
    if constexpr (KEEP) mb = softmax_prep(cur.mx, rescale, alpha);

    // ---- S(e+1) = K(e+1) Q^T, interleaved with P(e) = exp2(S(e) * c2 - mb) in bf16
    bf16x8_t pb[4];
    float rs = 0.0f;
    sn[0] = f32x16_t{};
    sn[1] = f32x16_t{};
    if constexpr (KEEP) {
#pragma unroll
      for (int st = 0; st < NQK; ++st) {
        qk_step(kt_next, sn, st);
#pragma unroll
        for (int u = 0; u < EPS; ++u) {
          const int j = st * EPS + u;
          const float pv_ = __builtin_amdgcn_exp2f(fmaf(sc[j >> 4][j & 15], c2, -mb));
          rs += pv_;
          pb[j >> 3][j & 7] = (__bf16)pv_;
        }
      }
    } else {
      // Skipped tile e: the registers of S(e) and P(e) are free, so the K fragments are
      // read SPF MFMAs ahead and the MFMAs issue without waiting on LDS.
      constexpr int SPF = NQK < 8 ? NQK : 8;
      bf16x8_t kf[SPF];
#pragma unroll
      for (int st = 0; st < SPF; ++st) kf[st] = k_frag(kt_next, st);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
      for (int st = 0; st < NQK; ++st) {
        const bf16x8_t kcur = kf[st % SPF];
        if (st + SPF < NQK) kf[st % SPF] = k_frag(kt_next, st + SPF);
        sn[st & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[st >> 1], sn[st & 1],
                                                             0, 0, 0);
      }
    }
    if constexpr (KEEP) {
      l_run += rs;
      // Keep P(e) here, next to the QK^T MFMAs it overlaps with: without a use at this
      // point the exp/convert work is sunk past the barrier into the P.V block.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" : : "v"(pb[ks]));
    }

    // ---- block maximum of tile e+1; stage V(e) and K(e+2) into LDS
    const int c_n = col_at(e + 1);
    const int cls_n = ldc_byte(a.cls, e + 1);
    nxt.mx = mask_max(sn, c_n, cls_n);
    if constexpr (GATE) {
      const float wm = wave_max(nxt.mx);
      if (lane == 0) sRed[(i + 1) & 1][wave] = wm;
    }
    if (KEEP || cur.any) ST::template store<VROW>(sV[i & 1], vr, tid);
    if (e + 2 < e1) ST::template store<KROW>(sK[i & 1], kr, tid);
    __syncthreads();  // V(e), K(e+2) and the maxima of tile e+1 are visible

    // ---- loads of K(e+3) right away (its registers were just staged), so they have
    // the rest of this step and the next QK^T block to land even when tiles are skipped
    if (e + 3 < e1) stk.load(kr, krs, (uint32_t)col_at(e + 3) * k_tile_bytes);

    // ---- gate(e+1)
    if constexpr (GATE) {
      decide((i + 1) & 1, cls_n, nxt);
    } else {
      nxt.keep = nxt.any = true;
    }

    // ---- O^T += V(e)^T P(e)^T
    if constexpr (KEEP) pv(sV[i & 1], pb, rescale, alpha);

    // ---- loads of V(e+1), only if some head keeps it; staged before the next barrier
    if (nxt.any) stv.load(vr, vrs, (uint32_t)c_n * v_tile_bytes);
    count_export(e, cur);
  };

  if (e0 < e1) {
    // prologue: K(e0), K(e0+1) staged; S(e0) and its gate; loads of V(e0) and K(e0+2)
    stk.load(kr, krs, (uint32_t)col_at(e0) * k_tile_bytes);
    ST::template store<KROW>(sK[0], kr, tid);
    if (e0 + 1 < e1) {
      stk.load(kr, krs, (uint32_t)col_at(e0 + 1) * k_tile_bytes);
      ST::template store<KROW>(sK[1], kr, tid);
    }
    __syncthreads();
    sA[0] = f32x16_t{};
    sA[1] = f32x16_t{};
#pragma unroll
    for (int st = 0; st < NQK; ++st) qk_step(sK[0], sA, st);
    const int cls0 = ldc_byte(a.cls, e0);
    stA.mx = mask_max(sA, col_at(e0), cls0);
    if constexpr (GATE) {
      const float wm = wave_max(stA.mx);
      if (lane == 0) sRed[0][wave] = wm;
    }
    __syncthreads();  // maxima visible; every wave is done reading sK[0]
    if constexpr (GATE) {
      decide(0, cls0, stA);
    } else {
      stA.keep = stA.any = true;
    }
    if (stA.any) stv.load(vr, vrs, (uint32_t)col_at(e0) * v_tile_bytes);
    if (e0 + 2 < e1) stk.load(kr, krs, (uint32_t)col_at(e0 + 2) * k_tile_bytes);

    // Unrolled by two so the scores alternate between sA and sB without copies.
    int e = e0;
    for (; e + 2 < e1; e += 2) {
      if (stA.keep)
        step(std::true_type{}, e, sA, stA, sB, stB);
      else
        step(std::false_type{}, e, sA, stA, sB, stB);
      if (stB.keep)
        step(std::true_type{}, e + 1, sB, stB, sA, stA);
      else
        step(std::false_type{}, e + 1, sB, stB, sA, stA);
    }
    if (e + 1 < e1) {
      if (stA.keep)
        step(std::true_type{}, e, sA, stA, sB, stB);
      else
        step(std::false_type{}, e, sA, stA, sB, stB);
      sA[0] = sB[0];
      sA[1] = sB[1];
      stA = stB;
      ++e;
    }

    // ---- the last tile: softmax, stage its V, P.V
    const int i = e - e0;
    bf16x8_t pb[4];
    bool rescale = false;
    float alpha = 1.0f;
    if (stA.keep) {
      const float mb = softmax_prep(stA.mx, rescale, alpha);
      float rs = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float pv_ = __builtin_amdgcn_exp2f(fmaf(sA[j >> 4][j & 15], c2, -mb));
        rs += pv_;
        pb[j >> 3][j & 7] = (__bf16)pv_;
      }
      l_run += rs;
    }
    if (stA.any) ST::template store<VROW>(sV[i & 1], vr, tid);
    __syncthreads();
    if (stA.keep) pv(sV[i & 1], pb, rescale, alpha);
    count_export(e, stA);
  }

  // ---- epilogue: O = O^T / l, LSE = scale * m + ln l; one store per element
  float l0, l1;
  pair32(l_run, l0, l1);
  const float l_tot = l0 + l1;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < a.N) {
    if (a.lse && half == 0) {
      a.lse[((int64_t)b * a.Hq + hq) * a.N + qi] =
          l_tot > 0.0f ? m_run * a.scale + logf(l_tot) : -INFINITY;
    }
    const int64_t obase = (int64_t)b * a.sob + (int64_t)hq * a.soh + (int64_t)qi * a.son;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * dt + 8 * r + 4 * half;
        if constexpr (OUT_F32) {
          float* op = reinterpret_cast<float*>(a.out) + obase + d0;
          *reinterpret_cast<float4*>(op) =
              make_float4(o[dt][4 * r] * inv, o[dt][4 * r + 1] * inv, o[dt][4 * r + 2] * inv,
                          o[dt][4 * r + 3] * inv);
        } else {
          uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + obase + d0;
          u32x2_t w;
          const __bf16 v0 = (__bf16)(o[dt][4 * r] * inv), v1 = (__bf16)(o[dt][4 * r + 1] * inv);
          const __bf16 v2 = (__bf16)(o[dt][4 * r + 2] * inv), v3 = (__bf16)(o[dt][4 * r + 3] * inv);
          w[0] = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
          w[1] = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
          *reinterpret_cast<u32x2_t*>(op) = w;
        }
      }
  }
  if (a.stats && (wave & 1) == 0 && lane == 0) {
    unsigned long long* st = a.stats + ((int64_t)b * a.Hq + hq) * 2;
    atomicAdd(st, (unsigned long long)n_kept);
    atomicAdd(st + 1, (unsigned long long)n_skip);
  }
}

// Warp-specialised variant for packs of four heads. Per head, one producer wave owns the
// whole 64-row query tile: it computes S^T = K Q^T for both 32-row halves, takes the gate
// (the tile maximum is a wave reduction, with no exchange between waves), runs the
// softmax, and writes P in bf16 together with its rescale factors to LDS. One consumer
// wave of the same head accumulates O^T += V^T P^T for the 64 rows, one step behind.
// Waves h and h + 4 (producer and consumer of head h) share a SIMD, so the consumer's
// P.V MFMAs run beside the producer's softmax work. The consumers also stage every K and
// V tile (global loads into registers, then LDS), so the producers hold no staging
// registers.
template <int D, int MODE, bool OUT_F32>
__global__ __launch_bounds__(512) void bsfa_fwd_ws_kernel(const FwdArgs a) {
  constexpr int HPACK = 4;
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
  __shared__ bf16x8_t sP[2][HPACK][2][4][64];  // P^T operands: [buf][head][rh][ks][lane]
  __shared__ float sAlpha[2][HPACK][2][32];    // O rescale factor per row
  __shared__ uint32_t sFlag[2][HPACK];         // bit 0 keep, bits 1-2 rescale of rh 0/1
  __shared__ uint32_t sKeep[2];                // byte h: head h keeps the tile
  __shared__ float sL[HPACK][2][32];           // final row sums for the consumer

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const bool producer = wave < HPACK;
  const int h = wave & (HPACK - 1);  // head of the pack this wave serves

  const int packs = a.Hq / HPACK;
  const int P = a.B * packs;
  const int wg = blockIdx.x;
  int p, trank;
  if (P % 8 == 0) {
    const int per = P / 8;
    p = (wg % 8) * per + (wg / 8) % per;
    trank = wg / P;
  } else {
    p = wg % P;
    trank = wg / P;
  }
  const int b = p / packs, hp = p % packs;
  const int t = a.nqt - 1 - trank;
  const int hq = hp * HPACK + h;
  const int g = (hp * HPACK) / a.group;
  int qi[2];
  qi[0] = t * BLK + l32;
  qi[1] = t * BLK + 32 + l32;

  int e0 = ldc(a.row_ptr, t), e1 = ldc(a.row_ptr, t + 1);
  e0 = e0 < 0 ? 0 : (e0 > a.nnz ? (int)a.nnz : e0);
  e1 = e1 < e0 ? e0 : (e1 > a.nnz ? (int)a.nnz : e1);
  const int nkb = a.nqt;
  auto col_at = [&](int e) {
    const int c = ldc(a.col, e);
    return c < 0 ? 0 : (c > nkb ? nkb : c);
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

  // Keep decisions of the pack for tile slot s (all heads), after a barrier.
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
              // a select, not an and/or blend of the bits (see the lock-step kernel)
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
      bool any;
    };
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.0f, 0.0f};
    unsigned n_kept = 0, n_skip = 0;
    const float c2 = a.scale_log2;
    auto gate = [&](PState& st, int cls, int slot) {
      if constexpr (GATE) {
        const float tm = wave_max(fmaxf(st.mx[0], st.mx[1])) * a.scale;
        st.tmax = tm;
        st.keep = (cls & BSFA_CLS_FORCED) != 0 || tm >= tau;
        if (lane == 0) reinterpret_cast<volatile uint8_t*>(&sKeep[slot])[h] = st.keep ? 1 : 0;
      } else {
        st.keep = true;
      }
    };
    auto softmax_prep = [&](int rh, float mx, bool& rescale, float& alpha) -> float {
      float x0, x1;
      pair32(mx, x0, x1);
      const float m_new = fmaxf(m_run[rh], fmaxf(x0, x1));
      const bool grow =
          (m_run[rh] == -INFINITY) ? (m_new != -INFINITY) : ((m_new - m_run[rh]) * c2 > 8.0f);
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
    auto count_export = [&](int e, const PState& st) {
      if (st.keep) ++n_kept; else ++n_skip;
      if (EXPORT && lane == 0) {
        const int64_t idx = ((int64_t)b * a.Hq + hq) * a.nnz + e;
        a.tile_max[idx] = st.tmax;
        a.keep[idx] = st.keep ? 1 : 0;
      }
    };

    f32x16_t sA[2][2], sB[2][2];
    PState stA{{-INFINITY, -INFINITY}, 0.0f, false, false};
    PState stB{{-INFINITY, -INFINITY}, 0.0f, false, false};

    auto pstep = [&](auto keep_tag, const int e, f32x16_t (&sc)[2][2], PState& cur,
                     f32x16_t (&sn)[2][2], PState& nxt) {
      constexpr bool KEEP = decltype(keep_tag)::value;
      const int i = e - e0, buf = i & 1;
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
      const int c_n = col_at(e + 1);
      const int cls_n = ldc_byte(a.cls, e + 1);
      mask_max(sn, c_n, cls_n, nxt.mx);
      gate(nxt, cls_n, (i + 1) & 1);
      __syncthreads();  // P(e), V(e), K(e+2) and the keep bytes of tile e+1 are visible
      nxt.any = any_of((i + 1) & 1);
      count_export(e, cur);
    };

    if (e0 < e1) {
      __syncthreads();  // (1) K(e0), K(e0+1) staged by the consumers
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
      const int cls0 = ldc_byte(a.cls, e0);
      mask_max(sA, col_at(e0), cls0, stA.mx);
      gate(stA, cls0, 0);
      __syncthreads();  // (2) keep bytes of e0; every wave is done reading sK[0]
      stA.any = any_of(0);

      int e = e0;
      for (; e + 2 < e1; e += 2) {
        if (stA.keep) pstep(std::true_type{}, e, sA, stA, sB, stB);
        else pstep(std::false_type{}, e, sA, stA, sB, stB);
        if (stB.keep) pstep(std::true_type{}, e + 1, sB, stB, sA, stA);
        else pstep(std::false_type{}, e + 1, sB, stB, sA, stA);
      }
      if (e + 1 < e1) {
        if (stA.keep) pstep(std::true_type{}, e, sA, stA, sB, stB);
        else pstep(std::false_type{}, e, sA, stA, sB, stB);
#pragma unroll
        for (int rh = 0; rh < 2; ++rh)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) sA[rh][mt] = sB[rh][mt];
        stA = stB;
        ++e;
      }
      // the last tile: its softmax, then V(last) staged
      const int i = e - e0, buf = i & 1;
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
      count_export(e, stA);
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
          // whole-vector concatenation and bit cast (see the lock-step kernel)
          const i16x8_t cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, cat);
          o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p0, o[0][dt], 0, 0, 0);
          o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1, o[1][dt], 0, 0, 0);
        }
      }
    };

    if (e0 < e1) {
      // prologue, in step with the producers' barriers (1) and (2)
      stk.load(kr, krs, (uint32_t)col_at(e0) * k_tile_bytes);
      ST::template store<KROW>(sK[0], kr, ctid);
      if (e0 + 1 < e1) {
        stk.load(kr, krs, (uint32_t)col_at(e0 + 1) * k_tile_bytes);
        ST::template store<KROW>(sK[1], kr, ctid);
      }
      __syncthreads();  // (1)
      __syncthreads();  // (2)
      bool any_cur = any_of(0);
      if (any_cur) stv.load(vr, vrs, (uint32_t)col_at(e0) * v_tile_bytes);
      if (e0 + 2 < e1) stk.load(kr, krs, (uint32_t)col_at(e0 + 2) * k_tile_bytes);
      for (int e = e0; e + 1 < e1; ++e) {
        const int i = e - e0, buf = i & 1;
        if (i > 0) pv((i - 1) & 1);  // P.V of the tile before
        if (any_cur) ST::template store<VROW>(sV[buf], vr, ctid);
        if (e + 2 < e1) ST::template store<KROW>(sK[buf], kr, ctid);
        __syncthreads();
        if (e + 3 < e1) stk.load(kr, krs, (uint32_t)col_at(e + 3) * k_tile_bytes);
        const int c_n = col_at(e + 1);
        any_cur = any_of((i + 1) & 1);
        if (any_cur) stv.load(vr, vrs, (uint32_t)c_n * v_tile_bytes);
      }
      {
        const int i = e1 - 1 - e0, buf = i & 1;
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
      const float l_tot = e0 < e1 ? sL[h][rh][l32] : 0.0f;
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

template <int D, int MODE, bool OUT_F32>
hipError_t launch_ws_variant(const FwdArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * (a.Hq / 4) * a.nqt);
  hipLaunchKernelGGL((bsfa_fwd_ws_kernel<D, MODE, OUT_F32>), dim3(grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ws(const FwdArgs& a, bool out_f32, hipStream_t s) {
  if (a.tau == nullptr)
    return out_f32 ? launch_ws_variant<D, DENSE, true>(a, s) : launch_ws_variant<D, DENSE, false>(a, s);
  if (a.tile_max != nullptr)
    return out_f32 ? launch_ws_variant<D, GATED_EXPORT, true>(a, s)
                   : launch_ws_variant<D, GATED_EXPORT, false>(a, s);
  return out_f32 ? launch_ws_variant<D, GATED, true>(a, s) : launch_ws_variant<D, GATED, false>(a, s);
}

template <int D, int HPACK, int MODE, bool OUT_F32>
hipError_t launch_variant(const FwdArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * (a.Hq / HPACK) * a.nqt);
  hipLaunchKernelGGL((bsfa_fwd_kernel<D, HPACK, MODE, OUT_F32>), dim3(grid), dim3(128 * HPACK),
                     0, stream, a);
  return hipGetLastError();
}

template <int D, int HPACK, int MODE>
hipError_t launch_mode(const FwdArgs& a, bool out_f32, hipStream_t s) {
  return out_f32 ? launch_variant<D, HPACK, MODE, true>(a, s)
                 : launch_variant<D, HPACK, MODE, false>(a, s);
}

template <int D, int HPACK>
hipError_t launch_hpack(const FwdArgs& a, bool out_f32, hipStream_t s) {
  if (a.tau == nullptr) return launch_mode<D, HPACK, DENSE>(a, out_f32, s);
  if (a.tile_max != nullptr) return launch_mode<D, HPACK, GATED_EXPORT>(a, out_f32, s);
  return launch_mode<D, HPACK, GATED>(a, out_f32, s);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int hpack, bool out_f32, hipStream_t s) {
  switch (hpack) {
    case 4: return launch_ws<D>(a, out_f32, s);
    case 2: return launch_hpack<D, 2>(a, out_f32, s);
    default: return launch_hpack<D, 1>(a, out_f32, s);
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
