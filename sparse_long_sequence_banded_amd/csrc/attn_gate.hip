// Low-rank output gate of gated attention (SWA/Hybrid-RoPE blog, section 3, Gated Attention:
// the attention output goes through a 128-dimension bottleneck and then gates): for every token,
// o = its outputs over all heads (H*d values, head-major), z = W_down o (r values),
// out = o * sigmoid(W_up z), in place.
//
// General shapes: one wave gates 32 tokens (a workgroup of four waves, 128 tokens, shares the
// weights through LDS) with two chained products on 32x32x16 bf16 MFMA (fp32 sums):
//   Z^T [r x 32] = W_down [r x Hd] O^T [Hd x 32]   (A: W_down rows; B: the tokens' output rows)
//   G^T [Hd x 32] = W_up [Hd x r] Z^T [r x 32]     (B: Z^T straight from the first product's
//                                                  accumulators, rounded to bf16)
// The accumulator layout gives lane half hh the bottleneck rows 4hh + {0..3} and 8 + 4hh + {0..3}
// of each 16-row step, so the second product's A operands (W_up rows) are read in that order.
// Every token is read and written by one wave only, so the update in place is safe.

#include "attn_args.h"
#include "mfma_util.h"

namespace longattn {
namespace {

using namespace mfma;

// LDS rows are padded by 16 bytes so that the 32 rows a wave reads land in different banks.
constexpr int kGateKChunk = 64;                  // W_down columns per staged chunk
constexpr int kGateDownRow = kGateKChunk + 8;    // padded row length (bf16)

template <int R>
__global__ __launch_bounds__(256) void gate_lowrank_kernel(GateArgs a) {
  constexpr int ZB = R / 32;  // 32-row blocks of Z^T
  constexpr int UPROW = R + 8;  // padded W_up row (bf16)
  // one buffer, used for W_down chunks [R][64] during the first product and for W_up row blocks
  // [32][R] during the second
  constexpr int kElems = (R * kGateDownRow > 32 * UPROW) ? R * kGateDownRow : 32 * UPROW;
  __shared__ __attribute__((aligned(16))) uint16_t wsm[kElems];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qj = lane & 31, hh = lane >> 5;
  const long tokens = (long)a.B * a.n;
  const long tok = ((long)blockIdx.x * 4 + wave) * 32 + qj;  // this lane's token (B operand col)
  const bool tok_ok = tok < tokens;
  const long tb = tok_ok ? tok / a.n : 0, ti = tok_ok ? tok % a.n : 0;
  const int Hd = a.H * a.d;
  // element e = h*d + c of this token's outputs
  auto optr = [&](int e) -> uint16_t* {
    return a.out + ((tb * a.H + e / a.d) * a.n + ti) * a.d + e % a.d;
  };

  // ---- Z^T = W_down O^T, W_down staged 64 columns at a time
  f32x16 z[ZB];
#pragma unroll
  for (int zb = 0; zb < ZB; ++zb)
#pragma unroll
    for (int r = 0; r < 16; ++r) z[zb][r] = 0.f;
  for (int k0 = 0; k0 < Hd; k0 += kGateKChunk) {
    // this chunk's output rows of the token (loaded before the barrier, used after it)
    u32x4 bo[kGateKChunk / 16];
#pragma unroll
    for (int ks = 0; ks < kGateKChunk / 16; ++ks) {
      bo[ks] = u32x4{0, 0, 0, 0};
      if (tok_ok && k0 + 16 * ks < Hd) bo[ks] = *reinterpret_cast<const u32x4*>(optr(k0 + 16 * ks + 8 * hh));
    }
    __syncthreads();  // the previous chunk is consumed
    for (int e = tid; e < R * (kGateKChunk / 8); e += 256) {
      const int row = e / (kGateKChunk / 8), c8 = e % (kGateKChunk / 8);
      u32x4 v = u32x4{0, 0, 0, 0};
      if (k0 + 8 * c8 < Hd) v = *reinterpret_cast<const u32x4*>(a.w_down + (long)row * Hd + k0 + 8 * c8);
      *reinterpret_cast<u32x4*>(&wsm[row * kGateDownRow + 8 * c8]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kGateKChunk / 16; ++ks)
#pragma unroll
      for (int zb = 0; zb < ZB; ++zb) {
        const u32x4 aw = *reinterpret_cast<const u32x4*>(&wsm[(32 * zb + qj) * kGateDownRow + 16 * ks + 8 * hh]);
        z[zb] = mfma_32x32x16(aw, bo[ks], z[zb]);
      }
  }
  // Z^T as bf16 B operands: step s (rows 16s .. 16s+15) uses accumulator block s/2, registers
  // 8(s%2) .. 8(s%2)+7
  uint32_t zp[ZB][8];
#pragma unroll
  for (int zb = 0; zb < ZB; ++zb)
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[zb][j] = pack_bf16x2(z[zb][2 * j], z[zb][2 * j + 1]);

  // ---- G^T = W_up Z^T, one 32-row block of the outputs at a time (W_up rows staged), then
  // the gate
  for (int ob = 0; ob < Hd; ob += 32) {
    // the outputs this lane gates in this block, loaded ahead of the barrier
    u32x2 ov[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      ov[q4] = u32x2{0, 0};
      if (tok_ok) ov[q4] = *reinterpret_cast<const u32x2*>(optr(ob + 8 * q4 + 4 * hh));
    }
    __syncthreads();
    for (int e = tid; e < 32 * (R / 8); e += 256) {
      const int row = e / (R / 8), c8 = e % (R / 8);
      *reinterpret_cast<u32x4*>(&wsm[row * UPROW + 8 * c8]) =
          *reinterpret_cast<const u32x4*>(a.w_up + (long)(ob + row) * R + 8 * c8);
    }
    __syncthreads();
    f32x16 g;
#pragma unroll
    for (int r = 0; r < 16; ++r) g[r] = 0.f;
    const uint16_t* wrow = &wsm[qj * UPROW];
#pragma unroll
    for (int s = 0; s < R / 16; ++s) {
      const int rb = 16 * s;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(wrow + rb + 4 * hh);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(wrow + rb + 8 + 4 * hh);
      const int zb = s >> 1, j0 = 4 * (s & 1);
      g = mfma_32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]},
                        u32x4{zp[zb][j0], zp[zb][j0 + 1], zp[zb][j0 + 2], zp[zb][j0 + 3]}, g);
    }
    if (!tok_ok) continue;
    // lane (token, hh) holds output rows ob + 8(j/4) + 4hh + j%4: four runs of 4 consecutive
    // elements of one head
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 w;
      w[0] = pack_bf16x2(bf16_lo(ov[q4][0]) * sigmoid_fast(g[4 * q4]),
                         bf16_hi(ov[q4][0]) * sigmoid_fast(g[4 * q4 + 1]));
      w[1] = pack_bf16x2(bf16_lo(ov[q4][1]) * sigmoid_fast(g[4 * q4 + 2]),
                         bf16_hi(ov[q4][1]) * sigmoid_fast(g[4 * q4 + 3]));
      *reinterpret_cast<u32x2*>(optr(ob + 8 * q4 + 4 * hh)) = w;
    }
  }
}

// The same gate when H*d = COLS*NW (NW <= 8) and r <= 128: one workgroup of NW waves gates
// TB blocks of 32 tokens, wave w owning the COLS output elements [COLS w, COLS w + COLS) of each
// token, so the launch has a workgroup per 32 TB tokens.
//   Z^T: wave w multiplies its COLS columns of W_down with its outputs (a split of the sum over
//   H*d), and the NW partial sums are added through LDS, one 32-row block of Z^T at a time.
//   G^T: wave w computes its COLS rows, then gates its own outputs.
// Each W_down and W_up fragment a wave loads serves its TB token blocks (two MFMAs at TB = 2),
// so the weights, which every workgroup reads in full from L2 with 16-byte loads scattered over
// 32 rows, cost half as much per token, and at 16K tokens the grid is one resident round.
// In the first product a lane's eight k-slots of 16-column step s are the columns
// 16s + 8hh + {0..7} (one 16-byte load each of outputs and of W_down).  In the second product
// the order of the output rows within a 32-row block is free: A's row qj = 8q + 4h' + e is taken
// as W_up row pi(qj) = 16(q/2) + 8h' + 4(q%2) + e, so lane half hh's accumulators hold rows
// 16(q/2) + 8hh + 4(q%2) + {0..3}: exactly the columns that lane loaded in steps 2b and 2b + 1.
// The outputs therefore stay in registers between the two products and are read from memory
// once.
template <int NW, int R, int COLS, int TB>
__global__ __launch_bounds__(NW * 64) void gate_lowrank_split_kernel(GateArgs a) {
  constexpr int ZB = R / 32;
  constexpr int KSW = COLS / 16;  // 16-column steps per wave
  // partial blocks are stored token-major: a token's 32 rows, padded to 36 floats so that the
  // 16-byte writes of 16 consecutive tokens hit distinct banks
  constexpr int TSTR = 36;
  constexpr int ZROW = R + 8;    // padded token row of Z (bf16)
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) float red[TB][NW * 32 * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t zt[TB][32 * ZROW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qj = lane & 31, hh = lane >> 5;
  const long tokens = (long)a.B * a.n;
  const int Hd = a.H * a.d;
  const int c0 = COLS * wave;
  const long head_stride = (long)a.n * a.d;

  // ---- this wave's outputs of token block k: columns c0 + 16s + 8hh + {0..7} of the lane's
  // token (8 consecutive elements stay in one head: d is a multiple of 16).  Element e sits in
  // head e / d at column e % d; the (head, column) pair is stepped by 16 columns per s rather
  // than divided out, and the loads go out together.  A lane past the last token reads token
  // 0's outputs: they only enter that lane's own column of the products, and nothing of it is
  // stored.
  bool tok_ok[TB];
  uint16_t* orow[TB][KSW];
  u32x4 of[TB][KSW];
#pragma unroll
  for (int k = 0; k < TB; ++k) {
    const long tok = ((long)blockIdx.x * TB + k) * 32 + qj;
    tok_ok[k] = tok < tokens;
    const long tb = tok_ok[k] ? tok / a.n : 0, ti = tok_ok[k] ? tok % a.n : 0;
    const int e0 = c0 + 8 * hh;
    int h = e0 / a.d, c = e0 - h * a.d;
    uint16_t* tok_base = a.out + (tb * a.H * a.n + ti) * a.d;
#pragma unroll
    for (int s = 0; s < KSW; ++s) {
      orow[k][s] = tok_base + h * head_stride + c;
      c += 16;
      if (c >= a.d) {
        c -= a.d;
        ++h;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < TB; ++k)
#pragma unroll
    for (int s = 0; s < KSW; ++s) of[k][s] = *reinterpret_cast<const u32x4*>(orow[k][s]);

  // W_up fragments of the second product's 32-row block b (A operands; A row qj is W_up row
  // pi(qj) of the block), loaded one block ahead of their products, the first block's during the
  // last reduction of the first product
  const int prow = 16 * (qj >> 4) + 8 * ((qj >> 2) & 1) + 4 * ((qj >> 3) & 1) + (qj & 3);
  constexpr int NB = COLS / 32;
  constexpr int RS = R / 16;
  const uint16_t* wup = a.w_up + (long)(c0 + prow) * R + 8 * hh;
  u32x4 wf[2][RS];

  // ---- Z^T = W_down O^T, one 32-row block at a time: this wave's partial sum over its columns
  // for every token block, then the NW partials added through LDS and stored as bf16 rows per
  // token.  The W_down fragments of block zb + 1 are loaded while block zb is multiplied and
  // reduced (measured 31.0 -> 29.2 us at 16K tokens x 1024 x r 128, with the early W_up loads
  // 27.5 us; a second reduction buffer, one barrier per block instead of two, changed nothing).
  const uint16_t* wdn = a.w_down + (long)qj * Hd + c0 + 8 * hh;
  u32x4 aw[2][KSW];
#pragma unroll
  for (int s = 0; s < KSW; ++s) aw[0][s] = *reinterpret_cast<const u32x4*>(wdn + 16 * s);
#pragma unroll
  for (int zb = 0; zb < ZB; ++zb) {
    if (zb + 1 < ZB) {
#pragma unroll
      for (int s = 0; s < KSW; ++s)
        aw[(zb + 1) & 1][s] =
            *reinterpret_cast<const u32x4*>(wdn + (long)32 * (zb + 1) * Hd + 16 * s);
    }
    f32x16 z[TB];
#pragma unroll
    for (int k = 0; k < TB; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) z[k][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KSW; ++s)
#pragma unroll
      for (int k = 0; k < TB; ++k) z[k] = mfma_32x32x16(aw[zb & 1][s], of[k][s], z[k]);
    if (zb == ZB - 1) {
#pragma unroll
      for (int s = 0; s < RS; ++s) wf[0][s] = *reinterpret_cast<const u32x4*>(wup + 16 * s);
    }
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      // registers 4j .. 4j+3 are rows 8j + 4hh + {0..3} of token qj
      float* mine = red[k] + (wave * 32 + qj) * TSTR + 4 * hh;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(mine + 8 * j) =
            make_float4(z[k][4 * j], z[k][4 * j + 1], z[k][4 * j + 2], z[k][4 * j + 3]);
    }
    __syncthreads();
    // thread e adds rows 4(e%8) .. +3 of token (e/8)%32 over the waves (in wave order) and stores
    // them as four bf16 (16-byte reads and 8-byte writes instead of one word at a time: 27.7 ->
    // 27.4 us at 16K tokens x 1024 x r 128, 27.3 -> 26.2 us at 32K tokens x 512, same bits)
    for (int e = tid; e < TB * 32 * 8; e += NT) {
      const int k = e >> 8, t = (e >> 3) & 31, j4 = e & 7;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4 p = *reinterpret_cast<const float4*>(red[k] + (w * 32 + t) * TSTR + 4 * j4);
        v.x += p.x;
        v.y += p.y;
        v.z += p.z;
        v.w += p.w;
      }
      u32x2 zw;
      zw[0] = pack_bf16x2(v.x, v.y);
      zw[1] = pack_bf16x2(v.z, v.w);
      *reinterpret_cast<u32x2*>(&zt[k][t * ZROW + 32 * zb + 4 * j4]) = zw;
    }
    __syncthreads();
  }
  // ---- G^T for this wave's rows, then the gate
  u32x4 zf[TB][R / 16];
#pragma unroll
  for (int k = 0; k < TB; ++k)
#pragma unroll
    for (int s = 0; s < R / 16; ++s)
      zf[k][s] = *reinterpret_cast<const u32x4*>(&zt[k][qj * ZROW + 16 * s + 8 * hh]);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b + 1 < NB) {
#pragma unroll
      for (int s = 0; s < RS; ++s)
        wf[(b + 1) & 1][s] = *reinterpret_cast<const u32x4*>(wup + (long)32 * (b + 1) * R + 16 * s);
    }
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      f32x16 g;
#pragma unroll
      for (int r = 0; r < 16; ++r) g[r] = 0.f;
#pragma unroll
      for (int s = 0; s < RS; ++s) g = mfma_32x32x16(wf[b & 1][s], zf[k][s], g);
      if (!tok_ok[k]) continue;
      // registers 4q .. 4q+3: rows c0 + 32b + 16(q/2) + 8hh + 4(q%2) + {0..3}, i.e. step
      // 2b + q/2, slots 4(q%2) .. 4(q%2)+3
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4& f = of[k][2 * b + (q >> 1)];
        const uint32_t w0 = (q & 1) ? f[2] : f[0], w1 = (q & 1) ? f[3] : f[1];
        u32x2 w;
        w[0] = pack_bf16x2(bf16_lo(w0) * sigmoid_fast(g[4 * q]),
                           bf16_hi(w0) * sigmoid_fast(g[4 * q + 1]));
        w[1] = pack_bf16x2(bf16_lo(w1) * sigmoid_fast(g[4 * q + 2]),
                           bf16_hi(w1) * sigmoid_fast(g[4 * q + 3]));
        *reinterpret_cast<u32x2*>(orow[k][2 * b + (q >> 1)] + 4 * (q & 1)) = w;
      }
    }
  }
}

#ifndef GATE_TB
#define GATE_TB 2
#endif
template <int NW, int COLS>
hipError_t launch_split(const GateArgs& a, long tokens, hipStream_t s) {
  constexpr int TB = GATE_TB;  // 32-token blocks per workgroup
  const dim3 grid((unsigned)((tokens + 32 * TB - 1) / (32 * TB))), block(NW * 64);
  switch (a.r) {
    case 32: hipLaunchKernelGGL((gate_lowrank_split_kernel<NW, 32, COLS, TB>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((gate_lowrank_split_kernel<NW, 64, COLS, TB>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((gate_lowrank_split_kernel<NW, 128, COLS, TB>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

#ifndef GATE_SPLIT_MAX
#define GATE_SPLIT_MAX 1024
#endif
hipError_t launch_gate_lowrank(const GateArgs& a, hipStream_t s) {
  const long tokens = (long)a.B * a.n;
  if (tokens <= 0) return hipSuccess;
  const int hd = a.H * a.d;
  if (hd % 128 == 0 && hd <= GATE_SPLIT_MAX && a.r <= 128) {
    switch (hd / 128) {
      case 1: return launch_split<1, 128>(a, tokens, s);
      case 2: return launch_split<2, 128>(a, tokens, s);
      case 3: return launch_split<3, 128>(a, tokens, s);
      case 4: return launch_split<4, 128>(a, tokens, s);
      case 5: return launch_split<5, 128>(a, tokens, s);
      case 6: return launch_split<6, 128>(a, tokens, s);
      case 7: return launch_split<7, 128>(a, tokens, s);
      case 8: return launch_split<8, 128>(a, tokens, s);
      default: break;
    }
  }
  const dim3 grid((unsigned)((tokens + 127) / 128));
  switch (a.r) {
    case 32: hipLaunchKernelGGL(gate_lowrank_kernel<32>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(gate_lowrank_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(gate_lowrank_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(gate_lowrank_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace longattn
