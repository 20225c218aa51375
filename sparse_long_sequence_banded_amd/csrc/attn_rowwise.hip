// fp32 sparse attention forward (one wave per query row) and the useful-entry counter.
//
// Both walk the candidate keys of a query row as row_sets.h describes (window, then global
// tokens, then layout blocks; global rows take every key; padded keys and duplicates dropped).
// The fp32 kernel is for the fp32 dtype only (small problems, every pattern combination).  The
// matrix-core kernels handle bf16.

#include "attn_args.h"
#include "row_sets.h"

namespace longattn {
namespace {

using namespace rowsets;

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
    if (col < d) {
      float y = acc[e] * inv;
      if (a.gate) {  // elementwise output gate: out *= sigmoid(gate logits)
        const float g = reinterpret_cast<const float*>(a.gate)[row * d + col];
        y = y / (1.f + expf(-g));
      }
      out[col] = y;
    }
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
