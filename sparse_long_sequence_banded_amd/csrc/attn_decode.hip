// Sliding-window decode over a key/value cache (bf16 or fp32).
//
// A few new query rows per sample attend the last `window` keys before and at their positions
// (the causal sliding window of the SWA decoder layers: SWAN-GPT summary, SWA-RoPE layers;
// SWA/Hybrid-RoPE blog, section 3).  There is little arithmetic per byte here (m <= 16 rows read
// the same window), so the kernels are built for the memory system.
//
// Head dims 64, 128 and 256 take decode_window_kernel: every lane loads 16-byte pieces of
// cache rows, a row spread over D*sizeof(T)/16 neighbouring lanes, so one load instruction of a
// wave reads 1 KiB of consecutive rows.  The loads are buffer loads against the (b, h) cache, so
// rows outside the cache read zeros without a branch.  Each lane issues its 16 K loads back to
// back (and its 16 V loads: up front for several new rows, right after the scores for one), so
// a wave keeps 16-32 KiB in flight; the per-row dot products are finished with a reduce-scatter
// across the lanes of a row.  Each wave takes the softmax
// of its own rows (wave max, weights, sum) and its weighted value sum; the waves of a workgroup
// are merged in LDS.  A workgroup that covers every position of the window writes the output
// rows directly; otherwise it writes a partial (unnormalised output, max, normaliser) per
// (row, chunk) and a small merge kernel combines the chunks.
//
// Other head dims take decode_generic_kernel (one cache row per thread, 256-position chunks,
// always partials + merge).  Arithmetic is fp32 (scores, weights, sums) on bf16 or fp32 inputs.

#include "attn_args.h"

namespace longattn {
namespace {

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kThreads = 256;

__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as floats.
__device__ __forceinline__ void load8(const uint16_t* p, float (&f)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
// 2 consecutive elements as floats.
__device__ __forceinline__ float2 load2(const uint16_t* p) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ float2 load2(const float* p) { return *reinterpret_cast<const float2*>(p); }

__device__ __forceinline__ void store_out(uint16_t* p, float x) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }

// ------------------------------------------------------------------ any head dim (d % 8 == 0)
// One workgroup: rows j < m of (b, h) against cache positions P0 .. P0 + 255 of the union of
// their windows.
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(DecodeArgs a) {
  __shared__ float qs[kDecodeMaxQueries * kDecodeMaxDim];  // the m query rows, fp32
  __shared__ float ps[kDecodeMaxQueries][kDecodeGenericChunk];  // scores, then weights
  __shared__ float red[kThreads * 2];                        // PV partial sums of one row
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int c = blockIdx.x % a.chunks;
  const long bh = blockIdx.x / a.chunks;
  const int b = (int)(bh / a.H);
  const int m = a.m, d = a.d;
  const int t0 = a.positions[b];
  const long first = (long)t0 - a.window + 1;      // window start of row 0 (may be negative)
  const long last = (long)t0 + m - 1;              // position of the last row
  const long P0 = first + (long)c * kDecodeGenericChunk;  // this chunk's first position
  const T* Qb = static_cast<const T*>(a.q) + bh * m * d;
  const T* Kb = static_cast<const T*>(a.k) + bh * (long)a.cache_len * d;
  const T* Vb = static_cast<const T*>(a.v) + bh * (long)a.cache_len * d;

  for (int i = t; i < m * d; i += kThreads) qs[i] = to_f32(Qb[i]);
  __syncthreads();

  // ---- scores: thread t takes position P0 + t
  const long pos = P0 + t;
  const bool in_cache = pos >= 0 && pos <= last && (a.ring || pos < a.cache_len);
  const long slot = in_cache ? (a.ring ? pos % a.cache_len : pos) : 0;
  float acc[kDecodeMaxQueries];
#pragma unroll
  for (int j = 0; j < kDecodeMaxQueries; ++j) acc[j] = 0.f;
  if (in_cache) {
    const T* krow = Kb + slot * d;
    for (int c0 = 0; c0 < d; c0 += 8) {
      float kf[8];
      load8(krow + c0, kf);
#pragma unroll
      for (int j = 0; j < kDecodeMaxQueries; ++j) {
        if (j < m) {
          const float* qj = qs + j * d + c0;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j] = __builtin_fmaf(qj[e], kf[e], acc[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kDecodeMaxQueries; ++j) {
    if (j < m) {
      const long tj = (long)t0 + j;  // position of row j: keys tj - window + 1 .. tj
      const bool ok = in_cache && pos <= tj && pos > tj - a.window;
      ps[j][t] = ok ? acc[j] * a.scale_log2 : -__builtin_inff();
    }
  }
  __syncthreads();

  // ---- per row: chunk max and weights 2^(s - max), chunk normaliser
  const long rows = (long)a.B * a.H * m;
  for (int j = wave; j < m; j += kThreads / 64) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kDecodeGenericChunk / 64; ++k) mx = fmaxf(mx, ps[j][lane + 64 * k]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < kDecodeGenericChunk / 64; ++k) {
      const float s = ps[j][lane + 64 * k];
      const float w = (s == -__builtin_inff()) ? 0.f : exp2f(s - mx);
      ps[j][lane + 64 * k] = w;
      l += w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      const long row = bh * m + j;
      float* pml = a.part + rows * a.chunks * d + (row * a.chunks + c) * 2;
      pml[0] = mx;
      pml[1] = l;
    }
  }
  __syncthreads();

  // ---- partial outputs: thread (g, cp) owns dims 2cp, 2cp+1 for positions g, g + G, ...
  const int tpr = d / 2;             // threads per value row
  const int G = kThreads / tpr;      // position groups
  const int g = t / tpr, cp = t % tpr;
  const bool active = g < G;
  float2 o[kDecodeMaxQueries];
#pragma unroll
  for (int j = 0; j < kDecodeMaxQueries; ++j) o[j] = make_float2(0.f, 0.f);
  if (active) {
    for (int k = g; k < kDecodeGenericChunk; k += G) {
      const long p = P0 + k;
      if (!(p >= 0 && p <= last && (a.ring || p < a.cache_len))) continue;  // not in the cache
      const long sl = a.ring ? p % a.cache_len : p;
      const float2 v = load2(Vb + sl * d + 2 * cp);
#pragma unroll
      for (int j = 0; j < kDecodeMaxQueries; ++j) {
        if (j < m) {
          const float w = ps[j][k];
          o[j].x = __builtin_fmaf(w, v.x, o[j].x);
          o[j].y = __builtin_fmaf(w, v.y, o[j].y);
        }
      }
    }
  }
  // reduce over the position groups, one row at a time
  for (int j = 0; j < m; ++j) {
    float2 oj = o[0];
#pragma unroll
    for (int jj = 1; jj < kDecodeMaxQueries; ++jj)
      if (jj == j) oj = o[jj];
    if (active) {
      red[2 * t] = oj.x;
      red[2 * t + 1] = oj.y;
    }
    __syncthreads();
    if (t < tpr) {
      float sx = 0.f, sy = 0.f;
      for (int gg = 0; gg < G; ++gg) {
        sx += red[2 * (gg * tpr + t)];
        sy += red[2 * (gg * tpr + t) + 1];
      }
      const long row = bh * m + j;
      float* po = a.part + (row * a.chunks + c) * d;
      po[2 * t] = sx;
      po[2 * t + 1] = sy;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ head dim 64, 128, 256
__device__ __forceinline__ void unpack16(const uint4& u, float (&f)[8]) {  // 8 bf16
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& u, float (&f)[4]) {  // 4 fp32
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}

// Reduce-scatter of NI values over groups of 2*OFF neighbouring lanes: at each step a lane keeps
// one half of its values (the upper half when its OFF bit is set), adds its partner's copy of
// that half, and sends the other half.  After the log2(LPR) steps a lane of a group of LPR
// lanes holds max(1, NI/LPR) complete sums: those of value indices seg*NI/LPR + u (LPR <= NI),
// or of index seg/(LPR/NI), shared by LPR/NI lanes (LPR > NI).
template <int OFF, int CNT, int NI>
__device__ __forceinline__ void reduce_scatter(float (&v)[NI], int seg) {
  if constexpr (OFF >= 1) {
    if constexpr (CNT > 1) {
      constexpr int H = CNT / 2;
      const bool up = (seg & OFF) != 0;
#pragma unroll
      for (int t = 0; t < H; ++t) {
        const float send = up ? v[t] : v[t + H];
        const float keep = up ? v[t + H] : v[t];
        v[t] = keep + __shfl_xor(send, OFF);
      }
      reduce_scatter<OFF / 2, H, NI>(v, seg);
    } else {
      v[0] += __shfl_xor(v[0], OFF);
      reduce_scatter<OFF / 2, 1, NI>(v, seg);
    }
  }
}

template <typename T, int D>
struct DecodeTile {
  static constexpr int kEPL = 16 / (int)sizeof(T);  // elements per 16-byte piece
  static constexpr int kLPR = D / kEPL;              // lanes per cache row
  static constexpr int kRPI = 64 / kLPR;             // rows per wave load instruction
  static constexpr int kNI = 16;                     // K (and V) loads per lane
  static constexpr int kPW = kNI * kRPI;             // positions per wave
  static constexpr int kVPL = kNI >= kLPR ? kNI / kLPR : 1;  // row sums per lane
  static constexpr int kDUP = kLPR > kNI ? kLPR / kNI : 1;   // lanes sharing a row sum
  static_assert(kLPR >= 1 && kLPR <= 64 && 64 % kLPR == 0, "head dim");
};

// Score of a query piece against a cache piece (16 bytes each), accumulated in fp32.
__device__ __forceinline__ float piece_dot(const uint4& q, const uint4& k, uint16_t) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float acc = 0.f;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x),
                                        __builtin_bit_cast(bf16x2, k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y),
                                        __builtin_bit_cast(bf16x2, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z),
                                        __builtin_bit_cast(bf16x2, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w),
                                        __builtin_bit_cast(bf16x2, k.w), acc, false);
  return acc;
}
__device__ __forceinline__ float piece_dot(const uint4& q, const uint4& k, float) {
  float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
  acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  return __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
}

// One workgroup: rows j < m of (b, h) against NW * PW consecutive positions of the union of their
// windows (chunk c).  Wave w takes positions P + w*PW .. P + w*PW + PW - 1; its lane (rsub, seg)
// loads piece seg of rows i*RPI + rsub, i < 16.  ONE (a single new row, m == 1): V is loaded
// once the scores are done, so only 16 loaded pieces are live at a time and two 8-wave
// workgroups fit on a compute unit; otherwise K and V stay loaded for all m rows.
template <typename T, int D, int NW, bool ONE>
__global__ __launch_bounds__(NW * 64) void decode_window_kernel(DecodeArgs a) {
  using Tl = DecodeTile<T, D>;
  constexpr int EPL = Tl::kEPL, LPR = Tl::kLPR, RPI = Tl::kRPI, NI = Tl::kNI, PW = Tl::kPW;
  constexpr int VPL = Tl::kVPL, DUP = Tl::kDUP;
  __shared__ float wsh[NW][PW];  // a wave's weights of one row
  __shared__ float osh[NW][D];   // a wave's weighted value sums of one row
  __shared__ float msh[NW], lsh[NW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = lane % LPR, rsub = lane / LPR;
  const int c = blockIdx.x % a.chunks;
  const long bh = blockIdx.x / a.chunks;
  const int b = (int)(bh / a.H);
  const int m = ONE ? 1 : a.m;
  const long t0 = a.positions[b];
  // Positions are handled as r = p - first, first = t0 - window + 1 (the first row's window
  // start); this lane's rows are r = rb + i*RPI.  Cache positions: lo <= r <= hi.
  const long first = t0 - a.window + 1;
  const int rb = c * (NW * PW) + wave * PW + rsub;
  const int lo = first < 0 ? (int)-first : 0;
  long hi_l = (long)a.window + m - 2;
  if (!a.ring) hi_l = hi_l < (long)a.cache_len - 1 - first ? hi_l : (long)a.cache_len - 1 - first;
  const int hi = hi_l < 0 ? -1 : (int)hi_l;
  // slot of r: ring: (first mod L) + r, less L past the end (r < L there); linear: first + r
  long fs = first;
  if (a.ring) {
    fs = first % a.cache_len;
    if (fs < 0) fs += a.cache_len;
  }
  const int sbase = (int)fs;  // linear: only used with r >= -first
  constexpr uint32_t kRowBytes = D * sizeof(T);
  const uint32_t nbytes = (uint32_t)a.cache_len * kRowBytes;
  const size_t head_off = (size_t)bh * a.cache_len * D;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(a.k) + head_off), (short)0, (int)nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(a.v) + head_off), (short)0, (int)nbytes, 0x00020000);
  const T* Qb = static_cast<const T*>(a.q) + bh * (long)m * D + seg * EPL;

  // Byte offsets of this lane's 16 pieces; rows outside the cache get an offset past the end
  // of the buffer, which reads zeros without touching memory.
  uint32_t off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = rb + i * RPI;
    int slot = sbase + r;
    if (a.ring && slot >= a.cache_len) slot -= a.cache_len;
    off[i] = (r >= lo && r <= hi) ? (uint32_t)slot * kRowBytes + seg * 16u : 0x80000000u;
  }
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, uint4 (&dst)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[i], 0, 0);
      dst[i] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  };
  const uint4 q0 = *reinterpret_cast<const uint4*>(Qb);  // row 0's piece, ahead of the K loads
  uint4 kr[NI], vr[NI];
  issue(krs, kr);
  if constexpr (!ONE) issue(vrs, vr);
  __builtin_amdgcn_sched_barrier(0);  // every load goes out before any of them is waited for

  const long rows = (long)a.B * a.H * m;
  const int base = LPR <= NI ? seg * VPL : seg / DUP;  // first row sum held by this lane
  for (int j = 0; j < m; ++j) {
    if constexpr (!ONE) {
      // keep the loaded pieces packed across rows: unpacked copies of all 32 would not fit in
      // registers, so the conversion is redone for every row instead of hoisted out of the loop
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        asm volatile("" : "+v"(kr[i].x), "+v"(kr[i].y), "+v"(kr[i].z), "+v"(kr[i].w));
        asm volatile("" : "+v"(vr[i].x), "+v"(vr[i].y), "+v"(vr[i].z), "+v"(vr[i].w));
      }
    }
    const uint4 qp = j == 0 ? q0 : *reinterpret_cast<const uint4*>(Qb + (long)j * D);
    float v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = piece_dot(qp, kr[i], T());
    if constexpr (ONE) {
      // the K pieces are dead from here: keep the V loads below this point so both never
      // occupy registers at once (the scores are pinned above it)
#pragma unroll
      for (int i = 0; i < NI; ++i) asm volatile("" : "+v"(v[i])::"memory");
      __builtin_amdgcn_sched_barrier(0);
      issue(vrs, vr);
      __builtin_amdgcn_sched_barrier(0);  // all 16 V loads go out back to back
    }
    reduce_scatter<LPR / 2, NI, NI>(v, seg);

    // ---- this wave's softmax of row j: scores in log2 units, wave max, weights, sum
    // row j (position t0 + j) sees r in [j, window - 1 + j], within the cache range
    const int rlo = lo > j ? lo : j;
    const int rhi = hi < a.window - 1 + j ? hi : a.window - 1 + j;
    float mx = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int r = rb + (base + u) * RPI;
      const bool ok = r >= rlo && r <= rhi;
      v[u] = ok ? v[u] * a.scale_log2 : -__builtin_inff();
      mx = fmaxf(mx, v[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const float w = (v[u] == -__builtin_inff()) ? 0.f : exp2f(v[u] - mx);
      if (seg % DUP == 0) {
        wsh[wave][(base + u) * RPI + rsub] = w;
        l += w;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    __syncthreads();

    // ---- weighted value sum of the wave's rows, reduced over the rows of a lane group
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float w = wsh[wave][i * RPI + rsub];
      float vf[EPL];
      unpack16(vr[i], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = __builtin_fmaf(w, vf[e], o[e]);
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], off);
    }
    if (rsub == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) osh[wave][seg * EPL + e] = o[e];
    }
    if (lane == 0) {
      msh[wave] = mx;
      lsh[wave] = l;
    }
    __syncthreads();

    // ---- merge the waves; write the row (one chunk) or the chunk's partial
    const int t = threadIdx.x;
    if (t < D) {
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, msh[w]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = (msh[w] == -__builtin_inff()) ? 0.f : exp2f(msh[w] - M);
        L = __builtin_fmaf(f, lsh[w], L);
        O = __builtin_fmaf(f, osh[w][t], O);
      }
      const long row = bh * m + j;
      if (a.chunks == 1) {
        store_out(static_cast<T*>(a.out) + row * D + t, L > 0.f ? O / L : 0.f);
        if (a.lse && t == 0) a.lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
      } else {
        a.part[(row * a.chunks + c) * D + t] = O;
        if (t == 0) {
          float* pml = a.part + rows * a.chunks * D + (row * a.chunks + c) * 2;
          pml[0] = M;
          pml[1] = L;
        }
      }
    }
    if (!ONE) __syncthreads();  // wsh, osh, msh, lsh are reused by the next row
  }
}

// Merge the chunks of every row: one wave per (b, h, j) row, four rows per workgroup.
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const long rows = (long)a.B * a.H * a.m;
  const long row = (long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int K = a.chunks, d = a.d;
  const float* po = a.part + row * K * d;
  const float* pml = a.part + rows * K * d + row * K * 2;
  float M = -__builtin_inff();
  for (int k = 0; k < K; ++k) M = fmaxf(M, pml[2 * k]);
  float L = 0.f;
  float acc[kDecodeMaxDim / 64];
#pragma unroll
  for (int e = 0; e < kDecodeMaxDim / 64; ++e) acc[e] = 0.f;
  if (M != -__builtin_inff()) {
    for (int k = 0; k < K; ++k) {
      const float mk = pml[2 * k];
      if (mk == -__builtin_inff()) continue;
      const float w = exp2f(mk - M);
      L += w * pml[2 * k + 1];
#pragma unroll
      for (int e = 0; e < kDecodeMaxDim / 64; ++e) {
        const int col = lane + 64 * e;
        if (col < d) acc[e] += w * po[(long)k * d + col];
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  T* orow = static_cast<T*>(a.out) + row * d;
#pragma unroll
  for (int e = 0; e < kDecodeMaxDim / 64; ++e) {
    const int col = lane + 64 * e;
    if (col < d) store_out(orow + col, acc[e] * inv);
  }
  if (a.lse && lane == 0) a.lse[row] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

}  // namespace

namespace {

template <typename T, int D>
constexpr int window_positions_per_wave() { return DecodeTile<T, D>::kPW; }

int positions_per_wave(bool bf16, int d) {
  switch (d) {
    case 64: return bf16 ? window_positions_per_wave<uint16_t, 64>() : window_positions_per_wave<float, 64>();
    case 128: return bf16 ? window_positions_per_wave<uint16_t, 128>() : window_positions_per_wave<float, 128>();
    case 256: return bf16 ? window_positions_per_wave<uint16_t, 256>() : window_positions_per_wave<float, 256>();
  }
  return 0;
}

template <typename T, int D, bool ONE>
void launch_window_rows(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.waves == 4)
    hipLaunchKernelGGL((decode_window_kernel<T, D, 4, ONE>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_window_kernel<T, D, 8, ONE>), grid, dim3(512), 0, s, a);
}

template <typename T, int D>
void launch_window(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.m == 1)
    launch_window_rows<T, D, true>(a, grid, s);
  else
    launch_window_rows<T, D, false>(a, grid, s);
}

template <typename T>
void launch_window_d(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.d) {
    case 64: launch_window<T, 64>(a, grid, s); break;
    case 128: launch_window<T, 128>(a, grid, s); break;
    default: launch_window<T, 256>(a, grid, s); break;
  }
}

}  // namespace

DecodeConfig decode_config(bool bf16, int d, long span, long bh) {
  DecodeConfig cfg;
  const int pw = positions_per_wave(bf16, d);
  if (pw == 0) {  // any other head dim: one cache row per thread, always partials + merge
    cfg.waves = 0;
    cfg.chunks = (span + kDecodeGenericChunk - 1) / kDecodeGenericChunk;
    cfg.merge = true;
    return cfg;
  }
  // 8 waves unless the window fits in 4 or fewer chunks would leave the GPU short of work
  // (fewer than 512 workgroups: two per compute unit)
  cfg.waves = span <= 4L * pw ? 4 : 8;
  cfg.chunks = (span + (long)cfg.waves * pw - 1) / ((long)cfg.waves * pw);
  if (cfg.waves == 8 && bh * cfg.chunks < 512) {
    cfg.waves = 4;
    cfg.chunks = (span + 4L * pw - 1) / (4L * pw);
  }
  cfg.merge = cfg.chunks > 1;
  return cfg;
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t s) {
  const long rows = (long)a.B * a.H * a.m;
  if (rows <= 0) return hipSuccess;
  const dim3 block(kThreads);
  const dim3 grid_p((unsigned)((long)a.B * a.H * a.chunks));
  const dim3 grid_m((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64)));
  if (a.waves > 0) {
    if (bf16)
      launch_window_d<uint16_t>(a, grid_p, s);
    else
      launch_window_d<float>(a, grid_p, s);
  } else if (bf16) {
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid_p, block, 0, s, a);
  } else {
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid_p, block, 0, s, a);
  }
  if (a.chunks > 1 || a.waves == 0) {
    if (bf16)
      hipLaunchKernelGGL(decode_merge_kernel<uint16_t>, grid_m, block, 0, s, a);
    else
      hipLaunchKernelGGL(decode_merge_kernel<float>, grid_m, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace longattn
