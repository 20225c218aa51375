// Backward pass of sparse attention, one wave per row (any pattern, bf16 or fp32 I/O, fp32
// arithmetic).
//
// With the forward's log-normaliser lse of each query row, the softmax weights are recomputed
// exactly (P = exp(s - lse)) and the gradients follow from the chain rule through the softmax:
// for an edge (i, j) with score s = scale * q_i . k_j,
//   P = exp(s - lse_i),  dP = dO_i . v_j,  dS = P * (dP - Drow_i),  Drow_i = dO_i . O_i,
//   dQ_i += scale * dS * k_j,   dK_j += scale * dS * q_i,   dV_j += P * dO_i.
// Three launches: Drow per row; dQ per query row over its key set; dK and dV per key column over
// the rows that attend it (row_sets.h lists both sides of every edge, each edge once).  Every
// sum has one owner, so there are no atomics and the results are deterministic.

#include "attn_args.h"
#include "row_sets.h"

namespace longattn {
namespace {

using namespace rowsets;

__device__ __forceinline__ float ldf(const float* p, long i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, long i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void stf(float* p, long i, float x) { p[i] = x; }
__device__ __forceinline__ void stf(uint16_t* p, long i, float x) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename T>
__device__ __forceinline__ float dot_rows(const T* x, const T* y, int d) {
  float acc = 0.f;
  for (int t = 0; t < d; ++t) acc = __builtin_fmaf(ldf(x, t), ldf(y, t), acc);
  return acc;
}

// Drow = dO . O for every row, one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BwdArgs g, long rows, int d) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* o = static_cast<const T*>(g.out) + row * d;
  const T* dO = static_cast<const T*>(g.dout) + row * d;
  float acc = 0.f;
  for (int c = lane; c < d; c += 64) acc = __builtin_fmaf(ldf(dO, c), ldf(o, c), acc);
  acc = wave_sum(acc);
  if (lane == 0) g.drow[row] = acc;
}

// dQ of one query row per wave: lanes take 64 candidate keys at a time.
template <typename T, int PER>
__global__ __launch_bounds__(256) void bwd_dq_rowwise_kernel(FwdArgs a, BwdArgs g, int d) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)a.B * a.H * a.n) return;
  const RowCtx r = make_row(a, row);
  const long bh = row / a.n;
  const T* q = static_cast<const T*>(static_cast<const void*>(a.q)) + row * d;
  const T* dO = static_cast<const T*>(g.dout) + row * d;
  const T* K = static_cast<const T*>(static_cast<const void*>(a.k)) + bh * a.n * d;
  const T* V = static_cast<const T*>(static_cast<const void*>(a.v)) + bh * a.n * d;
  const float lse = a.lse[row];
  const float drow = g.drow[row];
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (lse != -__builtin_inff()) {
    const long total = n_candidates(a, r);
    for (long c0 = 0; c0 < total; c0 += 64) {
      const long c = c0 + lane;
      const int j = (c < total) ? candidate_key(a, r, c) : -1;
      float ds = 0.f;
      if (j >= 0) {
        const float s = dot_rows(q, K + (long)j * d, d) * a.scale;
        const float p = expf(s - lse);
        const float dp = dot_rows(dO, V + (long)j * d, d);
        ds = p * (dp - drow);
      }
      for (int k = 0; k < 64; ++k) {
        const int jk = __shfl(j, k);
        if (jk < 0) continue;
        const float dsk = __shfl(ds, k);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int col = lane + 64 * e;
          if (col < d) acc[e] = __builtin_fmaf(dsk, ldf(K, (long)jk * d + col), acc[e]);
        }
      }
    }
  }
  T* dq = static_cast<T*>(g.dq) + row * d;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int col = lane + 64 * e;
    if (col < d) stf(dq, col, acc[e] * a.scale);
  }
}

// dK and dV of one key column per wave: lanes take 64 attending rows at a time.
template <typename T, int PER>
__global__ __launch_bounds__(256) void bwd_dkdv_rowwise_kernel(FwdArgs a, BwdArgs g, int d) {
  const int lane = threadIdx.x & 63;
  const long col = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= (long)a.B * a.H * a.n) return;
  const ColCtx c = make_col(a, col);
  const long bh = col / a.n;
  const T* Q = static_cast<const T*>(static_cast<const void*>(a.q)) + bh * a.n * d;
  const T* dO = static_cast<const T*>(g.dout) + bh * a.n * d;
  const T* kj = static_cast<const T*>(static_cast<const void*>(a.k)) + col * d;
  const T* vj = static_cast<const T*>(static_cast<const void*>(a.v)) + col * d;
  const float* lse = a.lse + bh * a.n;
  const float* drow = g.drow + bh * a.n;
  float ak[PER], av[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) ak[e] = av[e] = 0.f;

  // One chunk of up to 64 attending rows (i < 0: no row in this lane).
  auto chunk = [&](int i) {
    float p = 0.f, ds = 0.f;
    if (i >= 0) {
      const float s = dot_rows(Q + (long)i * d, kj, d) * a.scale;
      p = expf(s - lse[i]);
      const float dp = dot_rows(dO + (long)i * d, vj, d);
      ds = p * (dp - drow[i]);
    }
    for (int k = 0; k < 64; ++k) {
      const int ik = __shfl(i, k);
      if (ik < 0) continue;
      const float pk = __shfl(p, k), dsk = __shfl(ds, k);
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int cc = lane + 64 * e;
        if (cc < d) {
          av[e] = __builtin_fmaf(pk, ldf(dO, (long)ik * d + cc), av[e]);
          ak[e] = __builtin_fmaf(dsk, ldf(Q, (long)ik * d + cc), ak[e]);
        }
      }
    }
  };

  if (!c.padded) {
    if (c.is_global) {
      for (int c0 = 0; c0 < a.n; c0 += 64) chunk(c0 + lane < a.n ? c0 + lane : -1);
    } else {
      for (int c0 = 0; c0 < a.g; c0 += 64) chunk(c0 + lane < a.g ? c.gb[c0 + lane] : -1);
      for (int c0 = 0; c0 < c.n_band; c0 += 64) {
        const int idx = c0 + lane;
        chunk(idx < c.n_band ? column_band_row(a, c, idx) : -1);
      }
      if (a.layout) {
        const int nb = a.n / a.block, kb = c.j / a.block;
        for (int qb = 0; qb < nb; ++qb) {
          if (!layout_lists(a, c.h, qb, kb)) continue;
          for (int c0 = 0; c0 < a.block; c0 += 64) {
            const int i = qb * a.block + c0 + lane;
            chunk(c0 + lane < a.block && column_layout_row_ok(a, c, i) ? i : -1);
          }
        }
      }
    }
  }
  T* dk = static_cast<T*>(g.dk) + col * d;
  T* dv = static_cast<T*>(g.dv) + col * d;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int cc = lane + 64 * e;
    if (cc < d) {
      stf(dk, cc, ak[e] * a.scale);
      stf(dv, cc, av[e]);
    }
  }
}

template <typename T, int PER>
void launch_rowwise_bwd_t(const FwdArgs& a, const BwdArgs& g, int d, long grid, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_rowwise_kernel<T, PER>), dim3(grid), dim3(256), 0, s, a, g, d);
  hipLaunchKernelGGL((bwd_dkdv_rowwise_kernel<T, PER>), dim3(grid), dim3(256), 0, s, a, g, d);
}

}  // namespace

hipError_t launch_bwd_rowdot(const BwdArgs& g, long rows, int d, bool bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(bwd_rowdot_kernel<uint16_t>, grid, dim3(256), 0, s, g, rows, d);
  else
    hipLaunchKernelGGL(bwd_rowdot_kernel<float>, grid, dim3(256), 0, s, g, rows, d);
  return hipGetLastError();
}

hipError_t launch_bwd_rowwise(const FwdArgs& a, const BwdArgs& g, int d, bool bf16,
                              hipStream_t s) {
  const long rows = (long)a.B * a.H * a.n;
  if (rows <= 0) return hipSuccess;
  const long grid = (rows + 3) / 4;
  if (bf16) {
    if (d <= 64) launch_rowwise_bwd_t<uint16_t, 1>(a, g, d, grid, s);
    else if (d <= 128) launch_rowwise_bwd_t<uint16_t, 2>(a, g, d, grid, s);
    else if (d <= 256) launch_rowwise_bwd_t<uint16_t, 4>(a, g, d, grid, s);
    else return hipErrorInvalidValue;
  } else {
    if (d <= 64) launch_rowwise_bwd_t<float, 1>(a, g, d, grid, s);
    else if (d <= 128) launch_rowwise_bwd_t<float, 2>(a, g, d, grid, s);
    else if (d <= 256) launch_rowwise_bwd_t<float, 4>(a, g, d, grid, s);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace longattn
