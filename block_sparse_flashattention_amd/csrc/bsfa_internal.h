// Internal interface between the host library (bsfa_host.cpp) and the HIP kernels
// (bsfa_fwd.hip). Not part of the public C ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/bsfa.h"

namespace bsfa {

// Everything one forward launch needs, passed by value as the kernel argument.
struct FwdArgs {
  const uint16_t* q;  // bf16 bits [B, Hq, N, d]
  const uint16_t* k;  // bf16 bits [B, Hkv, N, d]
  const uint16_t* v;  // bf16 bits [B, Hkv, N, d]
  void* out;          // bf16 or fp32 [B, Hq, N, d]
  float* lse;         // fp32 [B, Hq, N] or null
  int64_t sqb, sqh, sqn;
  int64_t skb, skh, skn;
  int64_t svb, svh, svn;
  int64_t sob, soh, son;
  int32_t B, Hq, Hkv, N;
  int32_t nqt;    // ceil(N / 64)
  int32_t group;  // Hq / Hkv
  int32_t causal, window, n_global;
  int32_t pattern;             // some pattern primitive is set (else all pairs pass)
  int32_t dilation, block;
  int32_t dil_span;             // dilation * taps clamped to 2^31 - 1; 0 = no limit
  unsigned long long dil_bits;  // bits 0, s, 2s, ... below 64 for dilation s < 64
  const int32_t* row_ptr;  // CSR of allowed tiles, device
  const int32_t* col;
  const uint8_t* cls;
  int64_t nnz;
  const float* tau;        // [Hq] or null (dense path)
  float scale;             // softmax scale applied to q.k
  float scale_log2;        // scale * log2(e)
  unsigned long long* stats;  // [B*Hq*2] or null
  float* tile_max;            // [B*Hq*nnz] or null
  uint8_t* keep;              // [B*Hq*nnz] or null
};

// Everything one decode launch needs: one new query row per (sequence, query head)
// against a key/value cache, in splits of DEC_BPS key blocks per workgroup.
constexpr int DEC_BPS = 4;  // 64-key blocks per split (one workgroup)
constexpr int DEC_SPLIT_THREADS = 128;    // threads per split workgroup
constexpr int DEC_COMBINE_THREADS = 256;  // threads per combine workgroup

struct DecArgs {
  const uint16_t* q;        // bf16 bits [B, Hq, d]
  const uint16_t* k;        // bf16 bits [B, Hkv, Lmax, d]
  const uint16_t* v;        // bf16 bits [B, Hkv, Lmax, d]
  const int32_t* lengths;   // [B], valid cache rows per sequence (clamped to [0, Lmax])
  void* out;                // bf16 or fp32 [B, Hq, d]
  float* lse;               // fp32 [B, Hq] or null
  float* ws;                // per-split partials [B, Hq, nsplit, d + 1]
  int64_t sqb, sqh;
  int64_t skb, skh, skn;
  int64_t svb, svh, svn;
  int64_t sob, soh;
  int32_t B, Hq, Hkv, Lmax;
  int32_t group;            // Hq / Hkv, at most 32
  int32_t nkb;              // ceil(Lmax / 64)
  int32_t nsplit;           // ceil(nkb / DEC_BPS)
  int32_t causal, window, n_global;
  int32_t pattern;          // some pattern primitive is set (else all pairs pass)
  int32_t dilation, block, dil_span;
  int32_t random_ppm, random_seed;
  int32_t force_diag, force_global;
  unsigned long long dil_bits;
  const float* tau;         // [Hq] or null (dense path)
  float scale, scale_log2;
  unsigned long long* stats;  // [B*Hq*2] or null
  float* tile_max;            // [B*Hq*nkb] or null
  uint8_t* keep;              // [B*Hq*nkb] or null
};

// Launches the decode split kernel and the combine kernel on `stream`.
int launch_decode(const DecArgs& a, int d, bool out_f32, void* stream, const char** err);

// Bytes of the fixed device scratch that bsfa_decode_static uses in place of a workspace.
constexpr int64_t DEC_STATIC_SCRATCH_BYTES = BSFA_DECODE_STATIC_SCRATCH_BYTES;

// Device address of the fixed decode scratch on the device of `stream` (looked up once per
// device). 0 or a negative bsfa_status; *err receives a static message on failure.
int decode_static_scratch(void* stream, void** ptr, const char** err);

// Per-head threshold calibration from exported block maxima (bsfa_calib.hip).
struct CalibState {
  uint32_t prefix, mask;  // selected high bits of the order statistic's key so far
  uint32_t rank;          // wanted rank among the keys that match the prefix
  uint32_t count_eq;      // how often the selected key occurs
  uint32_t n, lo;         // eligible maxima; index of the lower order statistic
  uint32_t minkey;        // smallest key above the selected one
  uint32_t hi_same;       // both interpolation neighbours are the selected value
  double vidx, prev;      // numpy's virtual index and adjusted previous index
};

struct CalibArgs {
  const float* tile_max;   // [B, Hq, n_blocks] exported block maxima (scaled units)
  const uint8_t* keep;     // [B, Hq, n_blocks] keep bits of the gate-only pass
  int32_t B, Hq;
  int64_t n_blocks;
  double q;                // quantile in [0, 1]
  float* tau;              // [Hq] result
  uint32_t* hist;          // [Hq, 256] workspace
  CalibState* state;       // [Hq] workspace
};

int launch_calibrate(const CalibArgs& a, void* stream, const char** err);
int64_t calibrate_grid(int64_t B, int64_t Hq, int64_t n_blocks);

// Launches the forward kernel variant for head dim d, head pack hpack (query heads of
// one KV group sharing a workgroup: 4, 2 or 1, with 1, 2 or 4 query tiles each), gated
// (tau != null) or dense, bf16 or fp32 output.
// Returns 0 or a negative bsfa_status; *err receives a static message on failure.
int launch_fwd(const FwdArgs& a, int d, int hpack, bool out_f32, void* stream,
               const char** err);

// Device-to-host copy on `stream`, then synchronise the stream. 0 or BSFA_ERR_HIP.
int copy_to_host_sync(void* dst, const void* src, size_t bytes, void* stream,
                      const char** err);

}  // namespace bsfa
