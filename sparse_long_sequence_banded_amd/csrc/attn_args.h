// Internal launch arguments shared by the host dispatcher and the kernels (not public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace longattn {

constexpr int kMaxTableHeads = 256;  // heads with individual dilations carried in the args
constexpr int kKeyTile = 64;          // keys per K/V tile staged through LDS
constexpr int kGlobalChunk = 512;     // keys (forward) or rows (backward) per global-row workgroup
constexpr int kGlobalCap = 256;       // global tokens the bf16 kernels stage in LDS

enum Mode : int { kBand = 0, kLayout = 1, kGlobalRows = 2 };

// Scalar launch arguments.
struct FwdCore {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const int32_t* gidx;    // [B][g] or null
  const uint8_t* kpad;    // [B][n] or null
  const int32_t* layout;  // [H][n/block][max_kb] or null
  float* part;            // global-row partials: [B*H][g][chunks][D] o, then [..][2] (m, l)
  const uint16_t* gate;   // elementwise output-gate logits [B][H][n][d] (out *= sigmoid), or null
  int B, H, n, g;
  int wl, wr;             // window extents clamped to n; band_on == 0 means no window
  int band_on;
  int block, max_kb;
  int chunks;             // key chunks of the global-row partial workgroups
  int chunk_keys;         // keys per chunk
  int grid_rows;          // global-row partial workgroups in the attention launch
  float scale;            // softmax scale (> 0)
  float scale_log2;       // scale * log2(e)
  int tiles_per_b;        // main-kernel workgroups per batch sample
  int uniform_dil;        // > 0: every head has this dilation
  int head_tiles;         // > 0: every head takes this many main-kernel workgroups
  int fair_from;          // workgroups with blockIdx.x >= fair_from take the balancing priority
  int rows_by_xcd;        // global-row workgroups take the heads their XCD's main work ended on
};

// Passed by value to every kernel (kernarg segment, read through scalar loads).  Kernels that
// hand the scalars to lambdas copy the FwdCore part into a local first: a lambda that captured
// the whole argument by reference would make the compiler copy its tables to scratch memory.
struct FwdArgs : FwdCore {
  int tile_off[kMaxTableHeads + 1];  // prefix sums of workgroups per head (non-uniform case)
  uint8_t dil[kMaxTableHeads];
};

// Backward-pass pointers (the forward's q, k, v, lse, pattern and scale come in FwdArgs).
struct BwdArgs {
  const void* out;   // [B][H][n][d] forward output
  const void* dout;  // [B][H][n][d] gradient of the loss w.r.t. out
  void* dq;          // [B][H][n][d] outputs
  void* dk;
  void* dv;
  float* drow;       // [B][H][n] workspace: dO . O per row
  float* lse2;       // [B][H][n] workspace: lse in log2 units (matrix-core path)
};
// dQ; dK and dV together; or dK and dV in two passes (each recomputes the scores)
enum BwdKind : int { kBwdDQ = 0, kBwdDKV = 1, kBwdDK = 2, kBwdDV = 3 };

// Sliding-window decode over a key/value cache.
constexpr int kDecodeGenericChunk = 256;  // cache positions per workgroup, generic head dims
constexpr int kDecodeMaxQueries = 16;     // new rows per sample
constexpr int kDecodeMaxDim = 256;

struct DecodeArgs {
  const void* q;            // [B][H][m][d]
  const void* k;            // [B][H][cache_len][d]
  const void* v;
  void* out;                // [B][H][m][d]
  float* lse;               // [B][H][m] or null
  const int32_t* positions; // [B]
  float* part;              // partial outputs [B*H*m][chunks][d], then (max, sum) [..][2]
  int B, H, d, m;
  int window, cache_len, ring, chunks;
  int waves;                // waves per workgroup of the head-dim-specific kernel; 0: generic
  float scale_log2;
};

// Work split of a decode call: `chunks` workgroups per (b, h), each covering `waves` * (its
// positions per wave) consecutive positions (generic kernel: 256); `merge` = partials are
// written and combined by the merge kernel (needs workspace).
struct DecodeConfig {
  int waves = 0;
  long chunks = 1;
  bool merge = true;
};
DecodeConfig decode_config(bool bf16, int d, long span, long bh);

// LongT5 Transient-Global attention.
constexpr int kTgMaxRadius = 512;               // local radius limit of the kernels
constexpr int kTgMaxRl = kTgMaxRadius + 191;    // local relative positions a workgroup meets
constexpr int kTgMaxMd = 512;                   // max_distance limit
constexpr int kTgMaxDm = 4096;                  // d_model limit (a multiple of 64)

struct TgArgs {
  const uint16_t* q;      // [B][H][n][D]
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* sk;     // [B][H][G][D] global tokens' keys and values
  const uint16_t* sv;
  uint8_t* side_valid;    // [B][G]
  const uint8_t* kpad;    // [B][n] or null
  float* bias;            // [H][2rl+1 + 2md+1] per-head bias vectors (log2 units)
  uint16_t* out;          // [B][H][n][D]
  float* lse;             // [B][H][n] or null
  uint16_t* sk_out;       // side pass outputs
  uint16_t* sv_out;
  int B, H, n, D, dm, G, blk, radius, rl, md, nb;
  float scale_log2, eps;
};

// Low-rank output gate.
struct GateArgs {
  uint16_t* out;            // [B][H][n][d], gated in place
  const uint16_t* w_down;   // [r][H*d]
  const uint16_t* w_up;     // [H*d][r]
  int B, H, n, d, r;
};

// Launchers (defined next to their kernels).
int main_rows_per_workgroup(int mode, int d, int block);
// Optional events that record a kernel's own start and end (attached to its dispatch).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
hipError_t launch_attention(const FwdArgs& a, int d, int mode, long grid, hipStream_t s,
                            const LaunchEvents& ev);
hipError_t launch_global_combine(const FwdArgs& a, int d, hipStream_t s, const LaunchEvents& ev);

hipError_t launch_rowwise_f32(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_count_entries(const FwdArgs& a, int64_t* out, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_rowdot(const BwdArgs& g, long rows, int d, bool bf16, hipStream_t s);
hipError_t launch_bwd_rowwise(const FwdArgs& a, const BwdArgs& g, int d, bool bf16,
                              hipStream_t s);
// ev: null or three start/stop pairs (dQ kernel, dK/dV kernel, global-token combine)
hipError_t launch_bwd_mfma(const FwdArgs& a, const BwdArgs& g, int d, int mode, long grid,
                           hipStream_t s, const LaunchEvents* ev);
constexpr int kBwdMaxLayoutBlocks = 1024;  // matrix-core backward: n / block limit
hipError_t launch_tglobal_side(const TgArgs& a, const uint16_t* x, const float* gamma,
                               const uint16_t* wk, const uint16_t* wv, uint16_t* y,
                               hipStream_t s);
hipError_t launch_tglobal_attention(const TgArgs& a, const float* tab_local,
                                    const float* tab_side, hipStream_t s);
hipError_t launch_gate_lowrank(const GateArgs& a, hipStream_t s);

// Host: workgroups of `kernel` (launched with `threads` threads) that the device owning `stream`
// (the current device for the null stream) holds at once over all its CUs, taken once per device
// into `cache` (one cache per kernel); 0 when the runtime cannot say.
constexpr int kMaxDevices = 64;
inline long resident_capacity(const void* kernel, int threads, hipStream_t stream,
                              std::atomic<long> (&cache)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices) return 0;
  long cap = cache[dev].load(std::memory_order_relaxed);
  if (cap > 0) return cap;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cap = (long)per_cu * cus;
  cache[dev].store(cap, std::memory_order_relaxed);
  return cap;
}

// Host: the first workgroup (by blockIdx.x) that takes the balancing priority.  Every workgroup
// when the grid is a whole number of resident rounds (each round then ends at about the same time
// on every CU), else the last round only (the earlier rounds keep the hardware's oldest-first
// order, which spreads the remainder's workgroups over more CUs); none when the capacity is
// unknown.
inline int balancing_from(long grid, long cap) {
  if (cap <= 0) return 0x7fffffff;
  return grid % cap == 0 ? 0 : (int)std::max(0L, grid - cap);
}

}  // namespace longattn
