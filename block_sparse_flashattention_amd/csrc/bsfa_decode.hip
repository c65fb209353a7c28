// Block-sparse FlashAttention decode step for gfx950 (MI355X): one new query row per
// (sequence, query head) against a key/value cache.
//
// Method: token generation adds one token at a time and attends over the cached keys and
// values of all earlier tokens ("SAS: Sparse Attention Synthesizer", Challenge 2 "KV
// Cache Management" and Step 6). The block gate is the one of prefill (AI Radio episode
// "Block Sparse Flash Attention", "The paper's summary" and "The paper's improvements"),
// with the single new row as the query tile: every 64-key block of the cache gets the
// exact scores of the row, their maximum is compared with tau_h, and a block below it
// leaves the softmax and its V block is never loaded. The softmax over the kept keys is
// the renormalised one of prefill.
//
// Work decomposition
//   One workgroup = one (sequence b, KV head g, split s of DEC_BPS 64-key blocks); two
//   waves. The query heads of the KV group (G = Hq / Hkv <= 32) are the 32 columns of the
//   MFMA N dimension, and wave w owns keys [32 w, 32 w + 32) of every block: scores are
//   computed transposed, S^T = K Q^T (keys x heads), with the register layouts of the
//   prefill kernel. Decode reads every cached K row once and every kept V row once, so
//   it is bound by HBM bandwidth; the MFMA columns past G only cost idle matrix-core time.
//
//   Phase 1 streams the split's K blocks and keeps all of their scores in registers.
//   Each lane reduces the maximum of its head over its keys; the two waves exchange
//   their halves once through LDS, and the gate decides per head.
//   Phase 2 streams only the V blocks that some head of the group keeps. It accumulates
//   O^T += V^T P^T with P = exp(s - m), where m is the head's maximum over its kept blocks
//   of the split. That maximum is exact, so there is no running rescale.
//   The split then writes O / l and its log-sum-exp per head to the workspace, and a
//   second kernel merges the splits: LSE = log sum_s exp(LSE_s),
//   O = sum_s exp(LSE_s - LSE) O_s.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/bsfa.h"
#include "bsfa_internal.h"

namespace bsfa {

// Fixed device scratch for bsfa_decode_static, for callers that cannot allocate: the
// per-split partials live here instead of in a caller workspace. Every GPU the library
// runs on holds its own copy until the process ends. Host code never passes this name to
// a kernel (on the host it is only a stand-in for the symbol); it uses the device address
// that hipGetSymbolAddress returns for the device in question.
static __device__ __align__(256) unsigned char scratch[DEC_STATIC_SCRATCH_BYTES];

namespace {

#include "bsfa_device.h"

enum DecMode { DEC_DENSE = 0, DEC_GATED = 1, DEC_EXPORT = 2 };

// Workspace: the rows O_s [B, Hq, nsplit, d], then LSE_s [B, Hq, nsplit] in one block,
// so the combine reads each split's LSE from a compact array.
__device__ __forceinline__ float* ws_lse(const DecArgs& a, int d) {
  return a.ws + (int64_t)a.B * a.Hq * a.nsplit * d;
}

// SplitMix64 output for counter x (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The random primitive's choice for 64-token query block t and key block c.
__device__ __forceinline__ bool random_block(const DecArgs& a, int t, int c) {
  if (a.random_ppm <= 0) return false;
  const uint64_t counter = ((uint64_t)((uint32_t)a.random_seed & 0xFFFFFFu) << 40) |
                           ((uint64_t)(t & 0xFFFFF) << 20) | (uint64_t)(c & 0xFFFFF);
  const uint64_t threshold = ((uint64_t)(uint32_t)a.random_ppm << 32) / 1000000u;
  return (splitmix64(counter) >> 32) < threshold;
}

// Keys j0 + k, k in [0, 64), that row i may attend in a cache of n rows, as bit k
// (j0 a multiple of 64). Every primitive is a range or a residue class of k.
__device__ __forceinline__ uint64_t row_mask(const DecArgs& a, int n, int i, int j0) {
  const int r = i - j0;  // k of the row's own key
  uint64_t m = bits_below((int64_t)n - j0);
  if (a.causal) m &= bits_below((int64_t)r + 1);
  if (!a.pattern) return m;
  uint64_t p = (i < a.n_global) ? ~0ull : bits_below((int64_t)a.n_global - j0);
  if (a.window > 0)
    p |= bits_below((int64_t)r + a.window) & ~bits_below((int64_t)r - a.window + 1);
  if (a.dilation > 0) {
    const int st = a.dilation;
    const int off = ((r % st) + st) % st;  // keys k = off, off + st, ... below 64
    uint64_t dm = 0;
    if (off < 64) dm = (st >= 64 ? 1ull : a.dil_bits) << off;
    if (a.dil_span > 0)
      dm &= bits_below((int64_t)r + a.dil_span) & ~bits_below((int64_t)r - a.dil_span + 1);
    p |= dm;
  }
  if (a.block > 0) {
    const int64_t lo = (int64_t)(i / a.block) * a.block;
    p |= bits_below(lo + a.block - j0) & ~bits_below(lo - j0);
  }
  if (random_block(a, i / 64, j0 / 64)) p = ~0ull;
  return m & p;
}

template <int D, int MODE>
__global__ __launch_bounds__(DEC_SPLIT_THREADS) void bsfa_decode_kernel(const DecArgs a) {
  constexpr bool GATE = MODE != DEC_DENSE;
  constexpr bool EXPORT = MODE == DEC_EXPORT;
  constexpr int NT = DEC_SPLIT_THREADS;
  constexpr int KS = D / 16;  // 16-wide d steps of S^T = K Q^T
  constexpr int DT = D / 32;  // 32-row tiles of O^T along d
  constexpr int KROW = D + 8;
  constexpr int VROW = D + 32;

  __shared__ __attribute__((aligned(16))) uint16_t sK[BLK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BLK * VROW];
  __shared__ float sMax[2][DEC_BPS][32];
  __shared__ float sL[32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;

  const int s = blockIdx.x % a.nsplit;
  const int bg = blockIdx.x / a.nsplit;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  int n = ldc(a.lengths, b);
  n = n < 0 ? 0 : (n > a.Lmax ? a.Lmax : n);
  const int pos = n - 1;  // the new token's position
  const int nb = (n + BLK - 1) / BLK;
  const int c0 = s * DEC_BPS;
  int nblk = nb - c0;
  nblk = nblk < 0 ? 0 : (nblk > DEC_BPS ? DEC_BPS : nblk);
  const int G = a.group;
  const bool hv = l32 < G;  // this lane's column is a real query head
  const int hq = g * G + (hv ? l32 : 0);

  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = a.q + (int64_t)b * a.sqb + (int64_t)hq * a.sqh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = hv ? *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16 + half * 8) : bf16x8_t{};
  }
  const float tau = (GATE && hv) ? a.tau[hq] : 0.0f;

  // Buffer views end at the sequence's last valid row: cache rows at or past n (free
  // slots that may hold anything, NaN included) read as zeros, so a masked key's V row
  // cannot turn its zero weight into NaN inside the P.V product.
  const uint32_t k_bytes = n > 0 ? (uint32_t)(((int64_t)(n - 1) * a.skn + D) * 2) : 0u;
  const uint32_t v_bytes = n > 0 ? (uint32_t)(((int64_t)(n - 1) * a.svn + D) * 2) : 0u;
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
  u32x4_t kr[ST::CPT], vr[ST::CPT];

  // Allowed keys of each block of the split (wave-uniform).
  uint64_t bm[DEC_BPS];
#pragma unroll
  for (int bi = 0; bi < DEC_BPS; ++bi)
    bm[bi] = bi < nblk ? row_mask(a, n, pos, (c0 + bi) * BLK) : 0ull;
  // The first allowed block after bi (DEC_BPS if none).
  auto next_after = [&](int bi) {
    int nx = DEC_BPS;
#pragma unroll
    for (int bj = DEC_BPS - 1; bj >= 0; --bj)
      if (bj > bi && bm[bj] != 0ull) nx = bj;
    return nx;
  };

  // ---- phase 1: S^T of every allowed block (keys 32 * wave + [0, 32) x heads)
  const int kbase_el = l32 * KROW + half * 8 + wave * 32 * KROW;
  f32x16_t S[DEC_BPS];
  float hmax[DEC_BPS];
  {
    const int first = next_after(-1);
    if (first < DEC_BPS) stk.load(kr, krs, (uint32_t)(c0 + first) * k_tile_bytes);
  }
#pragma unroll
  for (int bi = 0; bi < DEC_BPS; ++bi) {
    S[bi] = f32x16_t{};
    hmax[bi] = -INFINITY;
    if (bm[bi] != 0ull) {
      ST::template store<KROW>(sK, kr, tid);
      __syncthreads();  // K(bi) visible
      const int nx = next_after(bi);
      if (nx < DEC_BPS) stk.load(kr, krs, (uint32_t)(c0 + nx) * k_tile_bytes);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(sK + kbase_el + ks * 16);
        S[bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[bi], 0, 0, 0);
      }
      if (bm[bi] != ~0ull) {
        // element i holds key 32 * wave + 8 * (i / 4) + 4 * half + i % 4 of the block
        const uint32_t w = (uint32_t)(bm[bi] >> (32 * wave)) >> (4 * half);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // a select, not an and/or blend of the bits (see the prefill kernel)
          const uint32_t bit = __builtin_amdgcn_ubfe(w, 8 * (i >> 2) + (i & 3), 1);
          S[bi][i] = bit ? S[bi][i] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[bi][i]);
      float x0, x1;
      pair32(mx, x0, x1);
      hmax[bi] = fmaxf(x0, x1);
      __syncthreads();  // every wave is done reading sK
    }
  }

  // ---- the gate: block maxima of both key halves, keep per head
  if (half == 0) {
#pragma unroll
    for (int bi = 0; bi < DEC_BPS; ++bi) sMax[wave][bi][l32] = hmax[bi];
  }
  __syncthreads();
  bool kp[DEC_BPS], anyk[DEC_BPS];
  float m_h = -INFINITY;  // raw maximum over the head's kept blocks of the split
  unsigned n_kept = 0, n_skip = 0;
#pragma unroll
  for (int bi = 0; bi < DEC_BPS; ++bi) {
    const int c = c0 + bi;
    const bool allowed = bm[bi] != 0ull;
    const float tm = fmaxf(sMax[0][bi][l32], sMax[1][bi][l32]);
    bool k = allowed && hv;
    if constexpr (GATE) {
      const bool forced = (a.force_diag && c == pos / BLK) ||
                          (a.force_global && (int64_t)c * BLK < (a.n_global < n ? a.n_global : n));
      k = k && (forced || tm * a.scale >= tau);
    }
    kp[bi] = k;
    anyk[bi] = __builtin_amdgcn_ballot_w64(k) != 0ull;
    if (k) m_h = fmaxf(m_h, tm);
    if (allowed) {
      if (k) ++n_kept; else ++n_skip;
    }
    if (EXPORT && wave == 0 && half == 0 && hv && c < a.nkb) {
      const int64_t idx = ((int64_t)b * a.Hq + hq) * a.nkb + c;
      a.tile_max[idx] = allowed ? tm * a.scale : -INFINITY;
      a.keep[idx] = k ? 1 : 0;
    }
  }
  if (a.stats && wave == 0 && half == 0 && hv && (n_kept | n_skip)) {
    unsigned long long* st = a.stats + ((int64_t)b * a.Hq + hq) * 2;
    atomicAdd(st, (unsigned long long)n_kept);
    atomicAdd(st + 1, (unsigned long long)n_skip);
  }

  // ---- phase 2: O^T += V^T P^T over the blocks some head keeps
  auto next_kept = [&](int bi) {
    int nx = DEC_BPS;
#pragma unroll
    for (int bj = DEC_BPS - 1; bj >= 0; --bj)
      if (bj > bi && anyk[bj]) nx = bj;
    return nx;
  };
  const float c2 = a.scale_log2;
  const float mb = (m_h == -INFINITY ? 0.0f : m_h) * c2;
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};
  float rs = 0.0f;
  const int jl = lane & 15;
  const int vbase_el = (4 * half + (jl >> 2)) * VROW + 16 * ((lane >> 4) & 1) + 4 * (jl & 3);
  {
    const int first = next_kept(-1);
    if (first < DEC_BPS) stv.load(vr, vrs, (uint32_t)(c0 + first) * v_tile_bytes);
  }
#pragma unroll
  for (int bi = 0; bi < DEC_BPS; ++bi) {
    if (anyk[bi]) {
      ST::template store<VROW>(sV, vr, tid);
      __syncthreads();  // V(bi) visible
      const int nx = next_kept(bi);
      if (nx < DEC_BPS) stv.load(vr, vrs, (uint32_t)(c0 + nx) * v_tile_bytes);
      bf16x8_t pb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // masked keys hold -inf (weight 0); a head that skips the block gets weight 0
        const float p = kp[bi] ? __builtin_amdgcn_exp2f(fmaf(S[bi][i], c2, -mb)) : 0.0f;
        rs += p;
        pb[i >> 3][i & 7] = (__bf16)p;
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* p0 = sV + vbase_el + 16 * (2 * wave + ks2) * VROW + 32 * dt;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(p0));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(p0 + 8 * VROW));
          // whole-vector concatenation and bit cast (see the prefill kernel)
          const i16x8_t cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, cat);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks2], o[dt], 0, 0, 0);
        }
      }
      __syncthreads();  // every wave is done reading sV
    }
  }

  // ---- merge the two key halves (wave 1 -> LDS -> wave 0), then write the partial
  float r0, r1;
  pair32(rs, r0, r1);
  const float lw = r0 + r1;  // this wave's sum of the head's weights
  float* sO = reinterpret_cast<float*>(sV);  // DT * 16 floats per lane of wave 1
  if (wave == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sO[(dt * 16 + r) * 64 + lane] = o[dt][r];
    if (half == 0) sL[l32] = lw;
  }
  __syncthreads();
  if (wave == 0) {
    const float l = lw + sL[l32];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (hv) {
      const int64_t part = ((int64_t)b * a.Hq + hq) * a.nsplit + s;
      float* wrow = a.ws + part * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = 32 * dt + 8 * r + 4 * half;
          float4 v4;
          v4.x = (o[dt][4 * r] + sO[(dt * 16 + 4 * r) * 64 + lane]) * inv;
          v4.y = (o[dt][4 * r + 1] + sO[(dt * 16 + 4 * r + 1) * 64 + lane]) * inv;
          v4.z = (o[dt][4 * r + 2] + sO[(dt * 16 + 4 * r + 2) * 64 + lane]) * inv;
          v4.w = (o[dt][4 * r + 3] + sO[(dt * 16 + 4 * r + 3) * 64 + lane]) * inv;
          *reinterpret_cast<float4*>(wrow + d0) = v4;
        }
      if (half == 0) ws_lse(a, D)[part] = l > 0.0f ? m_h * a.scale + logf(l) : -INFINITY;
    }
  }
}

// Merge the splits of one (sequence, query head) for 32 of its d outputs: each
// workgroup is one (sequence, head, 32-wide slice of d). Eight groups of 32 lanes take
// interleaved splits, each lane one output element, with several independent loads in
// flight; the group sums meet in LDS.
constexpr int COMBINE_THREADS = DEC_COMBINE_THREADS;
constexpr int COMBINE_GROUPS = COMBINE_THREADS / 32;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(COMBINE_THREADS) void bsfa_decode_combine(const DecArgs a) {
  constexpr int SLICES = D / 32;
  constexpr int UNROLL = 16;
  __shared__ float sAcc[COMBINE_GROUPS][33];
  __shared__ float sMx[COMBINE_THREADS / 64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = tid >> 5, el = tid & 31;
  const int64_t bh = blockIdx.x / SLICES;
  const int slice = blockIdx.x % SLICES;
  const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq);
  const int d = slice * 32 + el;
  const float* base = a.ws + bh * a.nsplit * D;
  const float* lse_s = ws_lse(a, D) + bh * a.nsplit;

  // the largest split LSE
  float mx = -INFINITY;
  for (int s = tid; s < a.nsplit; s += COMBINE_THREADS) mx = fmaxf(mx, lse_s[s]);
  mx = wave_max(mx);
  if (lane == 0) sMx[wave] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < COMBINE_THREADS / 64; ++w) mx = fmaxf(mx, sMx[w]);

  float acc = 0.0f, tot = 0.0f;
  if (mx != -INFINITY) {
    for (int s0 = grp; s0 < a.nsplit; s0 += COMBINE_GROUPS * UNROLL) {
      float ls[UNROLL], val[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int s = s0 + u * COMBINE_GROUPS;
        const bool ok = s < a.nsplit;
        ls[u] = ok ? lse_s[s] : -INFINITY;
        val[u] = base[(int64_t)(ok ? s : 0) * D + d];
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        // a split with no kept key has LSE -inf and weight 0 (its O_s row is 0 too)
        const float wgt = ls[u] == -INFINITY ? 0.0f : expf(ls[u] - mx);
        tot += wgt;
        acc = fmaf(wgt, val[u], acc);
      }
    }
  }
  sAcc[grp][el] = acc;
  if (el == 0) sAcc[grp][32] = tot;
  __syncthreads();
  if (tid < 32) {
    float v = 0.0f, t = 0.0f;
#pragma unroll
    for (int g = 0; g < COMBINE_GROUPS; ++g) {
      v += sAcc[g][el];
      t += sAcc[g][32];
    }
    const float val = t > 0.0f ? v / t : 0.0f;
    const int64_t o = (int64_t)b * a.sob + (int64_t)h * a.soh + d;
    if constexpr (OUT_F32)
      reinterpret_cast<float*>(a.out)[o] = val;
    else
      reinterpret_cast<__bf16*>(a.out)[o] = (__bf16)val;
    if (a.lse && slice == 0 && el == 0) a.lse[bh] = t > 0.0f ? mx + logf(t) : -INFINITY;
  }
}

template <int D, int MODE>
hipError_t launch_split(const DecArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hkv * a.nsplit);
  hipLaunchKernelGGL((bsfa_decode_kernel<D, MODE>), dim3(grid), dim3(DEC_SPLIT_THREADS), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecArgs& a, bool out_f32, hipStream_t s) {
  hipError_t e;
  if (a.tau == nullptr)
    e = launch_split<D, DEC_DENSE>(a, s);
  else if (a.tile_max != nullptr)
    e = launch_split<D, DEC_EXPORT>(a, s);
  else
    e = launch_split<D, DEC_GATED>(a, s);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hq * (D / 32));
  const dim3 block(COMBINE_THREADS);
  if (out_f32)
    hipLaunchKernelGGL((bsfa_decode_combine<D, true>), dim3(grid), block, 0, s, a);
  else
    hipLaunchKernelGGL((bsfa_decode_combine<D, false>), dim3(grid), block, 0, s, a);
  return hipGetLastError();
}

// Device address of `scratch` on each device, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int decode_static_scratch(void* stream, void** ptr, const char** err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return BSFA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = "device index out of range for the fixed decode scratch";
    return BSFA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // look the symbol up with the stream's device current, then restore the caller's
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || p == nullptr) {
      *err = e != hipSuccess ? hipGetErrorString(e) : "no device address for the scratch";
      return BSFA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BSFA_OK;
}

int launch_decode(const DecArgs& a, int d, bool out_f32, void* stream, const char** err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = d == 64 ? launch_decode_d<64>(a, out_f32, s)
                               : launch_decode_d<128>(a, out_f32, s);
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return BSFA_ERR_HIP;
  }
  return BSFA_OK;
}

}  // namespace bsfa
