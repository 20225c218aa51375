// fp32 sparse attention forward (one wave per query row) and the useful-entry counter.
//
// Both walk the same candidate list of a query row, in this order, keeping a candidate only if
// it is not padded and was not listed earlier:
//   global row:     every position (a global token attends the whole sequence; Longformer hub
//                   page, section 2; Big Bird reading notes, section 3.2.3);
//   any other row:  the window keys i + dil*t, t in [-win_left, win_right], inside [0, n)
//                   (Big Bird notes, section 3.2.1; dilation as on the Longformer hub page,
//                   section 2), then the global tokens, then the keys of the listed layout
//                   blocks (Big Bird notes, sections 3.2.2 and 3.3).
// Duplicates are dropped by testing membership in the earlier sets, so each (query, key) edge is
// counted once, as in the graph view of sparse attention (Big Bird notes, section 3.1).
//
// The fp32 kernel is for the fp32 dtype only (small problems, every pattern combination).  The
// matrix-core kernels handle bf16.

#include "attn_args.h"

namespace longattn {
namespace {

struct RowCtx {
  int b, h, i, dl;
  bool is_global;
  int t_lo, n_band;  // window keys i + dl * (t_lo + c), c < n_band
  int n_lay;         // listed layout blocks (slots, including unused ones)
  const int* lay_row;
  const int* gb;
  const uint8_t* pad;
};

__device__ __forceinline__ bool sorted_contains(const int* v, int len, int x) {
  int lo = 0, hi = len - 1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int y = v[mid];
    if (y == x) return true;
    if (y < x) lo = mid + 1; else hi = mid - 1;
  }
  return false;
}

__device__ __forceinline__ int floor_div(int a, int b) {  // b > 0
  int q = a / b;
  if ((a % b != 0) && (a < 0)) --q;
  return q;
}

__device__ RowCtx make_row(const FwdArgs& a, long row) {
  RowCtx r;
  r.i = (int)(row % a.n);
  const long bh = row / a.n;
  r.h = (int)(bh % a.H);
  r.b = (int)(bh / a.H);
  r.dl = a.uniform_dil > 0 ? a.uniform_dil : a.dil[r.h];
  r.gb = a.gidx ? a.gidx + (long)r.b * a.g : nullptr;
  r.pad = a.kpad ? a.kpad + (long)r.b * a.n : nullptr;
  r.is_global = a.g > 0 && sorted_contains(r.gb, a.g, r.i);
  r.t_lo = 0;
  r.n_band = 0;
  if (a.band_on) {
    const int t_lo = max(-a.wl, -floor_div(r.i, r.dl));
    const int t_hi = min(a.wr, floor_div(a.n - 1 - r.i, r.dl));
    r.t_lo = t_lo;
    r.n_band = max(0, t_hi - t_lo + 1);
  }
  r.n_lay = 0;
  r.lay_row = nullptr;
  if (a.layout) {
    const int nb = a.n / a.block;
    r.lay_row = a.layout + ((long)r.h * nb + r.i / a.block) * a.max_kb;
    r.n_lay = a.max_kb;
  }
  return r;
}

__device__ __forceinline__ bool in_band(const FwdArgs& a, const RowCtx& r, int j) {
  if (!a.band_on) return false;
  const long dd = (long)j - r.i;
  if (dd % r.dl != 0) return false;
  const long t = dd / r.dl;
  return t >= -a.wl && t <= a.wr;
}

__device__ __forceinline__ long n_candidates(const FwdArgs& a, const RowCtx& r) {
  if (r.is_global) return a.n;
  return (long)r.n_band + a.g + (long)r.n_lay * a.block;
}

// Key of candidate c, or -1 if it is padded, out of range, or an earlier duplicate.
__device__ int candidate_key(const FwdArgs& a, const RowCtx& r, long c) {
  int j = -1;
  if (r.is_global) {
    j = (int)c;
  } else if (c < r.n_band) {
    j = r.i + r.dl * (r.t_lo + (int)c);
  } else if (c < (long)r.n_band + a.g) {
    j = r.gb[c - r.n_band];
    if (j < 0 || j >= a.n || in_band(a, r, j)) j = -1;
  } else {
    const long e = c - r.n_band - a.g;
    const int id = r.lay_row[e / a.block];
    const int nb = a.n / a.block;
    if (id < 0 || id >= nb) return -1;
    j = id * a.block + (int)(e % a.block);
    if (in_band(a, r, j) || (a.g > 0 && sorted_contains(r.gb, a.g, j))) j = -1;
  }
  if (j >= 0 && r.pad && r.pad[j]) j = -1;
  return j;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int PER>
__global__ __launch_bounds__(256) void rowwise_f32_kernel(FwdArgs a, int d) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)a.B * a.H * a.n) return;
  const RowCtx r = make_row(a, row);
  const long bh = row / a.n;
  const float* q = reinterpret_cast<const float*>(a.q) + row * d;
  const float* K = reinterpret_cast<const float*>(a.k) + bh * a.n * d;
  const float* V = reinterpret_cast<const float*>(a.v) + bh * a.n * d;
  const float scale = a.scale;

  float m = -__builtin_inff(), l = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;

  const long total = n_candidates(a, r);
  for (long c0 = 0; c0 < total; c0 += 64) {
    const long c = c0 + lane;
    const int j = (c < total) ? candidate_key(a, r, c) : -1;
    float s = -__builtin_inff();
    if (j >= 0) {
      const float* kj = K + (long)j * d;
      float dot = 0.f;
      for (int t = 0; t < d; ++t) dot = __builtin_fmaf(q[t], kj[t], dot);
      s = dot * scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == -__builtin_inff()) continue;  // nothing valid yet
    const float alpha = expf(m - m_new);
    const float pj = (j >= 0) ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(pj);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= alpha;
    m = m_new;
    for (int k = 0; k < 64; ++k) {
      const int jk = __shfl(j, k);
      if (jk < 0) continue;
      const float pk = __shfl(pj, k);
      const float* vj = V + (long)jk * d;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int col = lane + 64 * e;
        if (col < d) acc[e] = __builtin_fmaf(pk, vj[col], acc[e]);
      }
    }
  }
  float* out = reinterpret_cast<float*>(a.out) + row * d;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int col = lane + 64 * e;
    if (col < d) out[col] = acc[e] * inv;
  }
  if (a.lse && lane == 0) a.lse[row] = (l > 0.f) ? m + logf(l) : -__builtin_inff();
}

// E = sum over rows of the number of kept candidates, and the same sum over global rows only.
// One thread per row, workgroup-level sums, one 64-bit atomic add per counter per workgroup.
__global__ __launch_bounds__(256) void count_entries_kernel(FwdArgs a,
                                                            unsigned long long* out) {
  __shared__ unsigned long long part[2][4];
  const long row = (long)blockIdx.x * 256 + threadIdx.x;
  unsigned long long cnt = 0, cnt_g = 0;
  if (row < (long)a.B * a.H * a.n) {
    const RowCtx r = make_row(a, row);
    const long total = n_candidates(a, r);
    for (long c = 0; c < total; ++c) cnt += candidate_key(a, r, c) >= 0 ? 1 : 0;
    if (r.is_global) cnt_g = cnt;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cnt += __shfl_xor(cnt, o);
    cnt_g += __shfl_xor(cnt_g, o);
  }
  if ((threadIdx.x & 63) == 0) {
    part[0][threadIdx.x >> 6] = cnt;
    part[1][threadIdx.x >> 6] = cnt_g;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(out, part[0][0] + part[0][1] + part[0][2] + part[0][3]);
    atomicAdd(out + 1, part[1][0] + part[1][1] + part[1][2] + part[1][3]);
  }
}

__global__ void zero_u64_kernel(unsigned long long* p) {
  p[0] = 0ull;
  p[1] = 0ull;
}

}  // namespace

hipError_t launch_rowwise_f32(const FwdArgs& a, int d, hipStream_t s) {
  const long rows = (long)a.B * a.H * a.n;
  if (rows <= 0) return hipSuccess;
  const long grid = (rows + 3) / 4;
  if (d <= 64) hipLaunchKernelGGL(rowwise_f32_kernel<1>, dim3(grid), dim3(256), 0, s, a, d);
  else if (d <= 128) hipLaunchKernelGGL(rowwise_f32_kernel<2>, dim3(grid), dim3(256), 0, s, a, d);
  else if (d <= 256) hipLaunchKernelGGL(rowwise_f32_kernel<4>, dim3(grid), dim3(256), 0, s, a, d);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_count_entries(const FwdArgs& a, int64_t* out, hipStream_t s) {
  auto* o = reinterpret_cast<unsigned long long*>(out);
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, o);
  const long rows = (long)a.B * a.H * a.n;
  if (rows > 0)
    hipLaunchKernelGGL(count_entries_kernel, dim3((rows + 255) / 256), dim3(256), 0, s, a, o);
  return hipGetLastError();
}

}  // namespace longattn
