// Per-head threshold calibration on the GPU: tau_h is the linear-interpolated quantile of
// head h's eligible block maxima (Block Sparse Flash Attention, "The paper's
// improvements": thresholds learned once per layer and head from the distribution of
// block maxima on a small data set). The maxima come from the gate-only pass of the
// forward or decode kernels (tau = NaN, per-block export): a block is eligible when it
// is allowed (finite maximum) and not forced (keep bit 0, since NaN keeps forced blocks
// only).
//
// The quantile is exact. Each maximum maps to an order-preserving 32-bit key, and a radix
// select over 8-bit digits finds the order statistic at index floor(v) of the virtual
// index v = (n - 1) q in four histogram rounds. A fifth pass takes the smallest key
// above it when the next order statistic is a different value. The interpolation follows
// numpy's default ("linear") quantile step by step in fp64, so the result equals
// np.quantile on the same maxima.
//
// Kernels, all on the caller's stream: init, then four rounds of (histogram, select), then
// the minimum above the selected key, then the interpolation. Histograms are built per
// workgroup in LDS and merged with atomics; each select clears its head's histogram for
// the next round.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/bsfa.h"
#include "bsfa_internal.h"

namespace bsfa {
namespace {

#include "bsfa_device.h"

constexpr int CALIB_THREADS = 256;
constexpr int CALIB_CHUNK = CALIB_THREADS * 16;  // maxima one histogram workgroup reads

// Order-preserving unsigned key of a float (finite values and infinities).
__device__ __forceinline__ uint32_t key_of(float x) {
  return (uint32_t)f2ord(x) ^ 0x80000000u;
}
__device__ __forceinline__ float value_of(uint32_t k) { return ord2f((int)(k ^ 0x80000000u)); }

__device__ __forceinline__ bool eligible(const CalibArgs& a, int64_t i, float& x) {
  x = a.tile_max[i];
  return a.keep[i] == 0 && x > -INFINITY && x <= INFINITY;  // allowed, not forced, not NaN
}

__global__ __launch_bounds__(CALIB_THREADS) void calib_init(const CalibArgs a) {
  const int h = blockIdx.x;
  a.hist[(int64_t)h * 256 + threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    CalibState s{};
    s.minkey = 0xFFFFFFFFu;
    a.state[h] = s;
  }
}

// Histogram of digit `round` (bits 31-8r .. 24-8r) of the keys that match the head's
// selected prefix so far. One workgroup reads one chunk of one (batch, head) row.
__global__ __launch_bounds__(CALIB_THREADS) void calib_hist(const CalibArgs a, int round) {
  __shared__ uint32_t sh[256];
  const int64_t rows = (int64_t)a.B * a.Hq;
  const int64_t chunks = (a.n_blocks + CALIB_CHUNK - 1) / CALIB_CHUNK;
  const int64_t row = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  if (row >= rows) return;
  const int h = (int)(row % a.Hq);
  sh[threadIdx.x] = 0u;
  __syncthreads();
  const CalibState s = a.state[h];
  const int shift = 24 - 8 * round;
  const int64_t e0 = chunk * CALIB_CHUNK;
  const int64_t e1 = e0 + CALIB_CHUNK < a.n_blocks ? e0 + CALIB_CHUNK : a.n_blocks;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += CALIB_THREADS) {
    float x;
    if (!eligible(a, row * a.n_blocks + e, x)) continue;
    const uint32_t k = key_of(x);
    if ((k & s.mask) == s.prefix) atomicAdd(&sh[(k >> shift) & 255u], 1u);
  }
  __syncthreads();
  const uint32_t c = sh[threadIdx.x];
  if (c) atomicAdd(&a.hist[(int64_t)h * 256 + threadIdx.x], c);
}

// Picks the digit whose bucket holds the wanted rank and clears the histogram. Round 0
// also counts the head's eligible maxima and places the virtual index.
__global__ __launch_bounds__(256) void calib_select(const CalibArgs a, int round) {
#pragma clang fp contract(off)
  __shared__ uint32_t cum[257];
  const int h = blockIdx.x, t = threadIdx.x;
  uint32_t* hist = a.hist + (int64_t)h * 256;
  const uint32_t c = hist[t];
  hist[t] = 0u;
  cum[t + 1] = c;
  if (t == 0) cum[0] = 0u;
  __syncthreads();
  if (t == 0)
    for (int i = 1; i <= 256; ++i) cum[i] += cum[i - 1];  // exclusive starts, then total
  __syncthreads();
  CalibState s = a.state[h];
  if (round == 0) {
    s.n = cum[256];
    if (s.n == 0) {
      if (t == 0) a.state[h] = s;
      return;
    }
    // numpy's virtual index for the linear method, (n - 1) q, and its neighbouring
    // indices: both the last one at or past n - 1, both 0 below 0.
    const double n = (double)s.n;
    const double v = (double)(s.n - 1) * a.q;
    s.vidx = v;
    if (v >= n - 1.0) {
      s.lo = s.n - 1;
      s.prev = -1.0;
      s.hi_same = 1;
    } else if (v < 0.0) {
      s.lo = 0;
      s.prev = 0.0;
      s.hi_same = 1;
    } else {
      s.prev = floor(v);
      s.lo = (uint32_t)s.prev;
    }
    s.rank = s.lo;
  } else if (s.n == 0) {
    return;
  }
  if (c > 0 && cum[t] <= s.rank && s.rank < cum[t] + c) {
    const int shift = 24 - 8 * round;
    s.rank -= cum[t];
    s.prefix |= (uint32_t)t << shift;
    s.mask |= 255u << shift;
    if (round == 3) s.count_eq = c;
    a.state[h] = s;
  }
}

// The smallest key above the selected one, per head (the next order statistic when the
// selected value does not repeat).
__global__ __launch_bounds__(CALIB_THREADS) void calib_min_above(const CalibArgs a) {
  __shared__ uint32_t sm[CALIB_THREADS / 64];
  const int64_t rows = (int64_t)a.B * a.Hq;
  const int64_t chunks = (a.n_blocks + CALIB_CHUNK - 1) / CALIB_CHUNK;
  const int64_t row = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  if (row >= rows) return;
  const int h = (int)(row % a.Hq);
  const CalibState s = a.state[h];
  uint32_t best = 0xFFFFFFFFu;
  if (s.n > 0) {
    const int64_t e0 = chunk * CALIB_CHUNK;
    const int64_t e1 = e0 + CALIB_CHUNK < a.n_blocks ? e0 + CALIB_CHUNK : a.n_blocks;
    for (int64_t e = e0 + threadIdx.x; e < e1; e += CALIB_THREADS) {
      float x;
      if (!eligible(a, row * a.n_blocks + e, x)) continue;
      const uint32_t k = key_of(x);
      if (k > s.prefix && k < best) best = k;
    }
  }
  // wave minimum, then across the workgroup's waves
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)best, off);
    best = o < best ? o : best;
  }
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = sm[0];
    for (int w = 1; w < CALIB_THREADS / 64; ++w) m = sm[w] < m ? sm[w] : m;
    if (m != 0xFFFFFFFFu) atomicMin(&a.state[h].minkey, m);
  }
}

// tau_h = numpy's linear interpolation between the two neighbouring order statistics,
// in fp64 without contraction, rounded to fp32. No eligible maximum gives -inf.
__global__ void calib_finalize(const CalibArgs a) {
#pragma clang fp contract(off)
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= a.Hq) return;
  const CalibState s = a.state[h];
  if (s.n == 0) {
    a.tau[h] = -INFINITY;
    return;
  }
  const double lo = (double)value_of(s.prefix);
  double hi = lo;
  // the next order statistic: the same value while it repeats, else the smallest above
  if (!s.hi_same && s.rank + 1 >= s.count_eq) hi = (double)value_of(s.minkey);
  const double g = s.vidx - s.prev;  // numpy's gamma, from its adjusted previous index
  const double d = hi - lo;
  double r = lo + d * g;
  if (g >= 0.5) r = hi - d * (1.0 - g);
  a.tau[h] = __double2float_rn(r);
}

}  // namespace

int launch_calibrate(const CalibArgs& a, void* stream, const char** err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(calib_init, dim3(a.Hq), dim3(CALIB_THREADS), 0, s, a);
  const int64_t chunks = (a.n_blocks + CALIB_CHUNK - 1) / CALIB_CHUNK;
  const int64_t grid = (int64_t)a.B * a.Hq * chunks;
  if (grid > 0) {
    for (int round = 0; round < 4; ++round) {
      hipLaunchKernelGGL(calib_hist, dim3((unsigned)grid), dim3(CALIB_THREADS), 0, s, a, round);
      hipLaunchKernelGGL(calib_select, dim3(a.Hq), dim3(256), 0, s, a, round);
    }
    hipLaunchKernelGGL(calib_min_above, dim3((unsigned)grid), dim3(CALIB_THREADS), 0, s, a);
  }
  hipLaunchKernelGGL(calib_finalize, dim3((a.Hq + 63) / 64), dim3(64), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = hipGetErrorString(e);
    return BSFA_ERR_HIP;
  }
  return BSFA_OK;
}

int64_t calibrate_grid(int64_t B, int64_t Hq, int64_t n_blocks) {
  return B * Hq * ((n_blocks + CALIB_CHUNK - 1) / CALIB_CHUNK);
}

}  // namespace bsfa
