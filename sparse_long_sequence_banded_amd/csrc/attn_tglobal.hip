// LongT5 Transient-Global attention on gfx950 (LongT5 guide: Transient-Global attention, the
// block and side helpers, relative position encoding).
//
// Global tokens.  The sequence is cut into blocks of k tokens (the trailing incomplete block
// merges into the one before it: G = max(1, n / k) global tokens, block(i) = min(i / k, G - 1)).
// Global token g is the sum of the embeddings of the block's non-padded tokens, RMS-normalised
// with the layer's weight (the T5 layer norm), then projected with the attention's key and value
// weights.  Two kernels: tg_aggregate_kernel (one workgroup per (b, g): block sum, RMS norm, the
// normalised row stored in bf16) and tg_project_kernel (the product with the bf16 weights on
// matrix cores).
//
// Attention.  Query i attends the local keys |i - j| <= radius (not padded) and every valid
// global token, all in one softmax, with T5 relative-position bias: table[bucket(j - i)][h] for
// local keys, table_side[bucket(g - block(i))][h] for global tokens.  The bucket of a distance
// saturates beyond max_distance, so tg_bias_kernel expands the two tables, once per call, into
// per-head vectors over the relative positions a workgroup can meet (log2 units, fp64 bucket
// decisions); tg_attn_kernel keeps them in LDS.  A local tile reads its bias at an offset that is
// a constant per register; a global-token tile whose distances to all of a wave's blocks are
// saturated adds one constant.
//
// The attention kernel is the forward kernel's scheme without dilation or layouts: a wave owns
// 32 query rows (Q fragments in registers), 64-row K/V tiles (local keys, then global tokens)
// stream through two LDS stages by direct buffer loads, S^T = K Q^T and O^T += V^T P^T on
// 32x32x16 bf16 MFMA, and the softmax keeps a lazily moved per-row reference (weights stay at
// or below 2^16 of it).

#include <type_traits>

#include "attn_args.h"
#include "mfma_util.h"

namespace longattn {
namespace {

using namespace mfma;

constexpr float kLog2eT = 1.44269504088896340736f;
constexpr float kRefSlack = 8.f;  // move a row's reference when its max exceeds it by > 2^8
constexpr float kTgFastWeightSum = 65536.f;  // fast path: a lane's 16 weights of a half sum to <= 2^16

// T5's bidirectional bucket of rel = key position - query position (fp64 decisions).
__device__ int t5_bucket(int rel, int nb, int md) {
  const int half = nb / 2;
  const int base = rel > 0 ? half : 0;
  const int a = rel < 0 ? -rel : rel;
  const int exact = half / 2;
  if (a < exact) return base + a;
  const double x = log((double)a / (double)exact) / log((double)md / (double)exact) *
                   (double)(half - exact);
  int off = exact + (int)floor(x);
  if (off > half - 1) off = half - 1;
  return base + off;
}

// Per-head bias vectors (log2 units): local[h][rel + RL] for |rel| <= RL and
// side[h][rel + md] for |rel| <= md (side distances are clamped to +-md by the kernel).
__global__ void tg_bias_kernel(TgArgs a, const float* tab_local, const float* tab_side) {
  const int h = blockIdx.y;
  const int L = 2 * a.rl + 1, S = 2 * a.md + 1;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < L + S; e += gridDim.x * blockDim.x) {
    float v;
    if (e < L) v = tab_local[t5_bucket(e - a.rl, a.nb, a.md) * a.H + h];
    else v = tab_side[t5_bucket(e - L - a.md, a.nb, a.md) * a.H + h];
    a.bias[(long)h * (L + S) + e] = v * kLog2eT;
  }
}

// Block sums and RMS norm: y[b][g][c] (bf16) and side_valid[b][g].  One wave per (b, g); lane l
// sums the 8-column groups l, l + 64, ... (KPG groups) over the block's rows with 16-byte loads,
// ROWS rows at a time with every load in flight (a padded row is read and weighted by 0; with
// one group per lane, 16 rows: a default 16-token block in one round of loads, global-token pass
// 12.5 -> 12.3 us at d_model 512, same bits).
template <int KPG>
__global__ __launch_bounds__(64) void tg_aggregate_kernel(TgArgs a, const uint16_t* x,
                                                         const float* gamma, uint16_t* y) {
  constexpr int ROWS = KPG == 1 ? 16 : (KPG == 2 ? 8 : (KPG == 4 ? 4 : 2));
  const int g = blockIdx.x % a.G;
  const int b = blockIdx.x / a.G;
  const int lane = threadIdx.x;
  const int i0 = g * a.blk;
  const int i1 = (g == a.G - 1) ? a.n : min(a.n, i0 + a.blk);  // the tail merges into the last
  const uint8_t* pad = a.kpad ? a.kpad + (long)b * a.n : nullptr;
  const int ng = a.dm / 8;
  const uint16_t* xb = x + (long)b * a.n * a.dm;
  float sum[KPG][8];
#pragma unroll
  for (int u = 0; u < KPG; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[u][e] = 0.f;
  bool anyv = false;
  for (int i = i0; i < i1; i += ROWS) {
    u32x4 xv[ROWS][KPG];
    float wt[ROWS];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      const int row = min(i + k, i1 - 1);
      wt[k] = (i + k < i1 && (pad == nullptr || pad[row] == 0)) ? 1.f : 0.f;
#pragma unroll
      for (int u = 0; u < KPG; ++u) {
        const int cg = lane + 64 * u;
        xv[k][u] = cg < ng ? *reinterpret_cast<const u32x4*>(xb + (long)row * a.dm + 8 * cg)
                           : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      anyv = anyv || wt[k] != 0.f;
#pragma unroll
      for (int u = 0; u < KPG; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[u][2 * e] = __builtin_fmaf(wt[k], bf16_lo(xv[k][u][e]), sum[u][2 * e]);
          sum[u][2 * e + 1] = __builtin_fmaf(wt[k], bf16_hi(xv[k][u][e]), sum[u][2 * e + 1]);
        }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < KPG; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(sum[u][e], sum[u][e], ss);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.f / sqrtf(ss / (float)a.dm + a.eps);
  uint16_t* yrow = y + ((long)b * a.G + g) * a.dm;
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const int cg = lane + 64 * u;
    if (cg >= ng) continue;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pack_bf16x2(sum[u][2 * e] * inv * gamma[8 * cg + 2 * e],
                         sum[u][2 * e + 1] * inv * gamma[8 * cg + 2 * e + 1]);
    *reinterpret_cast<u32x4*>(yrow + 8 * cg) = w;
  }
  // the valid flag is the same in every lane (the row weights are uniform)
  if (lane == 0) a.side_valid[(long)b * a.G + g] = (uint8_t)anyv;
}

// side_k / side_v [B][H][G][d] (bf16) = y [B*G][dm] (bf16) times W [dm][H*d] (bf16), on
// 32x32x16 bf16 MFMA with fp32 sums.  One wave makes a 32 x 32 output tile of one matrix.  Per
// 256-deep k chunk the W tile (256 x 32) and the y tile (32 x 256) go straight to LDS with
// 16-byte buffer loads (no register staging, every load in flight); the wave then reads its B
// operands with the transposing LDS read and its A operands with 8-byte LDS reads.  The y tile's
// 16-byte chunk c of row r sits at position c ^ r of the row, so the 32 rows' reads of one chunk
// hit different banks.  The MFMA's k slots of lane half hh are k = 4hh + {0..3} and
// 8 + 4hh + {0..3} within each 16-deep step (the transposing read's order), and the A operands
// follow the same order.
constexpr int kProjTile = 32, kProjK = 256;
__global__ __launch_bounds__(64) void tg_project_kernel(TgArgs a, const uint16_t* y,
                                                       const uint16_t* wk, const uint16_t* wv) {
  constexpr int KSC = kProjK / 16;  // k-steps per chunk
  __shared__ __attribute__((aligned(1024))) uint16_t ws[kProjK][kProjTile];  // W[k][col] chunk
  __shared__ __attribute__((aligned(1024))) uint16_t ys[kProjTile][kProjK];  // y[row][k] chunk
  const int lane = threadIdx.x;
  const int qj = lane & 31, hh = lane >> 5;
  const long rows = (long)a.B * a.G;
  const int HD = a.H * a.D;
  const long r0 = (long)blockIdx.x * kProjTile;
  const int c0 = blockIdx.y * kProjTile;
  const bool is_v = blockIdx.z == 1;
  // W rows are read from column c0 on, y rows from row r0 on; out-of-range reads give zeros
  const u32x4 wrs = buf_rsrc((is_v ? wv : wk) + c0,
                             (uint32_t)(((long)a.dm * HD - c0) * 2));
  const u32x4 yrs =
      buf_rsrc(y + r0 * a.dm, (uint32_t)(std::min(rows - r0, (long)kProjTile) * a.dm * 2));
  const uint32_t ws_lds = __builtin_amdgcn_readfirstlane(lds_addr(&ws[0][0]));
  const uint32_t ys_lds = __builtin_amdgcn_readfirstlane(lds_addr(&ys[0][0]));
  const int vi = lane & 15, vg = lane >> 4;
  const int trow = 4 * hh + (vi >> 2);
  const int tcol = 16 * (vg & 1) + 4 * (vi & 3);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int k0 = 0; k0 < a.dm; k0 += kProjK) {
    const int kc = min(kProjK, a.dm - k0);  // a multiple of 64
    if (k0 > 0) __syncthreads();  // the previous chunk is consumed
    // W: 16 rows of 64 bytes per load (lane l: row 16i + l/4, columns 8(l%4) .. + 7)
    for (int i = 0; i < kc / 16; ++i)
      lds_dma16(wrs, (uint32_t)(((k0 + 16 * i + (lane >> 2)) * HD + 8 * (lane & 3)) * 2),
                ws_lds + 1024 * i);
    // y: two rows per load; lane l fills position l%32 of row 2j + l/32 with that row's chunk
    // (l%32) ^ row (chunks past kc hold data that is never read)
    for (int j = 0; j < kProjTile / 2; ++j) {
      const int row = 2 * j + (lane >> 5);
      const int chunk = (lane & 31) ^ row;
      lds_dma16(yrs, (uint32_t)((row * a.dm + k0 + 8 * chunk) * 2), ys_lds + 1024 * j);
    }
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      if (16 * ks >= kc) break;
      // A: y[row qj][16ks + 4hh + {0..3}] (chunk 2ks) and y[row qj][16ks + 8 + 4hh + {0..3}]
      // (chunk 2ks + 1), the (8hh)-th bytes of those chunks
      const u32x2 lo = *reinterpret_cast<const u32x2*>(&ys[qj][8 * ((2 * ks) ^ qj) + 4 * hh]);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(&ys[qj][8 * ((2 * ks + 1) ^ qj) + 4 * hh]);
      // B: W[kb + 4hh + e][col] and W[kb + 8 + 4hh + e][col] for col = qj, by the transposing
      // read (lane l of 16-lane group G = l/16 names row 4*(l/32) + (l%16)/4 of the 4-row group
      // and 4 columns)
      const unsigned char* base = reinterpret_cast<const unsigned char*>(&ws[16 * ks][0]);
      const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(s16x4, base + trow * (2 * kProjTile) + 2 * tcol));
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(s16x4, base + (trow + 8) * (2 * kProjTile) + 2 * tcol));
      const u32x2 w0 = __builtin_bit_cast(u32x2, b0), w1 = __builtin_bit_cast(u32x2, b1);
      acc = mfma_32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, u32x4{w0[0], w0[1], w1[0], w1[1]},
                          acc);
    }
  }
  // C: lane (col qj, hh) holds rows 8(r/4) + 4hh + r%4 of the 32 x 32 tile
  const int col = c0 + qj;
  if (col >= HD) return;
  const int h = col / a.D, c = col % a.D;
  uint16_t* dst = is_v ? a.sv_out : a.sk_out;
  // (batch, global token) of the tile's first row, then stepped: one division per lane instead
  // of a 64-bit division per element (measured 10.0 -> 8.5 us at 1024 global tokens; a
  // 64 x 64 tile per four-wave workgroup with the whole 512-deep product staged at once, or a
  // second accumulation chain, gained nothing more)
  const int rbase = (int)r0;  // B * G < 2^31
  const int b0 = rbase / a.G, g0 = rbase - b0 * a.G;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int off = 8 * (r >> 2) + 4 * hh + (r & 3);
    if (rbase + off >= rows) continue;
    int b = b0, g = g0 + off;
    while (g >= a.G) {  // at most 31 / G + 1 steps
      g -= a.G;
      ++b;
    }
    dst[(((long)b * a.H + h) * a.G + g) * a.D + c] =
        __builtin_bit_cast(uint16_t, (__bf16)acc[r]);
  }
}

template <int D>
struct TgSmem {
  __attribute__((aligned(1024))) unsigned char stage_k[2][kKeyTile * D * 2];
  __attribute__((aligned(1024))) unsigned char stage_v[2][kKeyTile * D * 2];
  float bias_l[2 * kTgMaxRl + 1];
  float bias_s[2 * kTgMaxMd + 1];
};

template <int D>
__global__ __launch_bounds__(256) void tg_attn_kernel(TgArgs a) {
  constexpr int NW = 4, NT = 256, RW = 32, QT = NW * RW;
  constexpr int CH = D / 8, KS = D / 16, DB = D / 32;
  constexpr int NLOAD = 2 * CH, LPW = NLOAD / NW, RPB = 64 / CH;
  __shared__ TgSmem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qj = lane & 31, hh = lane >> 5;
  const int tiles_q = (a.n + QT - 1) / QT;
  const int Lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = Lid % tiles_q;
  const long bh = Lid / tiles_q;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int q0 = qt * QT;
  const uint16_t* Qb = a.q + bh * a.n * D;
  const uint8_t* pad = a.kpad ? a.kpad + (long)b * a.n : nullptr;
  const uint8_t* sval = a.side_valid + (long)b * a.G;

  // this lane's query row
  const int qpos = q0 + wave * RW + qj;
  const bool qok = qpos < a.n;
  const int qblk = min(qpos / a.blk, a.G - 1);
  // tiles: local keys first, then the global tokens
  const int q_last = min(q0 + QT, a.n) - 1;
  const int k_lo = max(0, q0 - a.radius), k_hi = min(a.n - 1, q_last + a.radius);
  const int n_local = (k_hi - k_lo + kKeyTile) / kKeyTile;
  const int n_side = (a.G + kKeyTile - 1) / kKeyTile;
  const int n_tiles = n_local + n_side;

  // ---- tile loading (waves 0-1: K blocks, waves 2-3: V blocks; 1 KB direct loads)
  const int mat = (wave * LPW) / CH;
  const int sub0 = (wave * LPW) % CH;
  auto ld_row = [&](int j) -> int { return (sub0 + j) * RPB + lane / CH; };
  auto ld_col = [&](int j) -> int {
    const int row = ld_row(j);
    return 8 * ((lane % CH) ^ (mat == 0 ? swz_k<D>(row) : swz_v<D>(row)));
  };
  uint32_t voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) voff[j] = (uint32_t)(ld_row(j) * D + ld_col(j)) * 2u;
  const uint16_t* lsrc = (mat == 0 ? a.k : a.v) + bh * a.n * D;
  const uint16_t* ssrc = (mat == 0 ? a.sk : a.sv) + bh * a.G * D;
  auto issue = [&](int si, int t) {
    unsigned char* stg = mat == 0 ? sm.stage_k[si] : sm.stage_v[si];
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stg + sub0 * 1024));
    u32x4 rs;
    if (t < n_local) {
      const int base = k_lo + t * kKeyTile;
      rs = buf_rsrc(lsrc + (long)base * D, (uint32_t)(a.n - base) * D * 2u);
    } else {
      const int base = (t - n_local) * kKeyTile;
      rs = buf_rsrc(ssrc + (long)base * D, (uint32_t)(a.G - base) * D * 2u);
    }
#pragma unroll
    for (int j = 0; j < LPW; ++j) lds_dma16(rs, voff[j], dst + 1024 * j);
  };
  if (n_tiles > 0) issue(0, 0);

  // Q fragments (B operands of S^T = K Q^T)
  u32x4 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = u32x4{0, 0, 0, 0};
    if (qok) qf[s] = *reinterpret_cast<const u32x4*>(Qb + (long)qpos * D + 16 * s + 8 * hh);
  }
  // bias vectors of this head
  const int L = 2 * a.rl + 1, S = 2 * a.md + 1;
  const float* bsrc = a.bias + (long)h * (L + S);
  for (int e = tid; e < L; e += NT) sm.bias_l[e] = bsrc[e];
  for (int e = tid; e < S; e += NT) sm.bias_s[e] = bsrc[L + e];
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" : : "v"(qf[s]));
  __syncthreads();

  // LDS read offsets (as in the forward kernel)
  const int ksw = swz_k<D>(qj);
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = qj * (2 * D) + (((2 * ks + hh) ^ ksw) * 16);
  const int vi = lane & 15, vg = lane >> 4;
  const int vrow0 = 4 * hh + (vi >> 2);
  const int vsw = swz_v<D>(vrow0);
  int voffs[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 4 * db + 2 * (vg & 1) + ((vi & 3) >> 1);
    voffs[db] = vrow0 * (2 * D) + ((chunk ^ vsw) * 16) + 8 * (vi & 1);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // l: sum of the bf16-rounded weights that multiply the value rows (the output's normaliser)
  float ref = 0.f, l_run = 0.f;
  bool has = false;
  const float c2 = a.scale_log2;
  const float ninf = neg_inf();
  // this wave's query rows and blocks (for skipping far tiles)
  const int w_first = q0 + wave * RW;
  const int w_last = min(w_first + RW - 1, a.n - 1);
  const bool wave_rows = w_first < a.n;
  const int wblk_lo = min(w_first / a.blk, a.G - 1), wblk_hi = min(w_last / a.blk, a.G - 1);

  auto tile = [&](int si, int t) {
    const unsigned char* sk_ = sm.stage_k[si];
    const unsigned char* sv_ = sm.stage_v[si];
    const bool local = t < n_local;
    const int base = local ? k_lo + t * kKeyTile : (t - n_local) * kKeyTile;
    // usable rows of the tile: local keys in range and not padded; valid global tokens
    bool ok;
    if (local) {
      const int pos = base + lane;
      ok = pos < a.n && (pad == nullptr || pad[pos] == 0);
    } else {
      const int g = base + lane;
      ok = g < a.G && sval[g] != 0;
    }
    const unsigned long long vmask = __ballot(ok);
    // scores S^T
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sk_ + koff[ks] + kb * 32 * (2 * D));
        sc[kb] = mfma_32x32x16(kf, qf[ks], sc[kb]);
      }
    }
    // Scores in log2 units plus bias, x = mul * y + off; register r of half kb is row
    // 32kb + 8(r/4) + 4hh + r%4.  Local tiles and near global-token tiles take a bias per element
    // (y = c2 s + bias, mul = 1, off = 0); a global-token tile whose distances to all of the
    // wave's blocks are saturated takes one constant, folded into the exponent (y = s, mul = c2,
    // off = that bias).
    float mul = 1.f, off = 0.f;
    if (local) {
      // bias_l index: (base + row) - qpos + rl, a per-lane base plus a constant per register
      const float* bl = sm.bias_l + (base - qpos + a.rl + 4 * hh);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[kb][r] = __builtin_fmaf(sc[kb][r], c2, bl[32 * kb + 8 * (r >> 2) + (r & 3)]);
    } else {
      const int far_pos = base - wblk_hi >= a.md;                  // every g - block >= md
      const int far_neg = base + kKeyTile - 1 - wblk_lo <= -a.md;  // every g - block <= -md
      if (far_pos || far_neg) {
        mul = c2;
        off = far_pos ? sm.bias_s[2 * a.md] : sm.bias_s[0];
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = base + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3) - qblk;
            const int idx = min(max(rel, -a.md), a.md) + a.md;
            sc[kb][r] = __builtin_fmaf(sc[kb][r], c2, sm.bias_s[idx]);
          }
      }
    }
    // masks (usable rows, and for local tiles the window |key - q| <= radius), only where some
    // key of the tile is excluded for some row of the wave
    bool need_mask = vmask != ~0ull || w_first + RW > a.n;
    if (local && !need_mask)
      need_mask = !(base >= w_last - a.radius && base + kKeyTile - 1 <= w_first + a.radius);
    if (need_mask) {
      unsigned long long m = vmask >> (4 * hh);
      if (local) {
        const int lo = qpos - a.radius - base - 4 * hh;
        const int hi = qpos + a.radius - base - 4 * hh;
        unsigned long long bm = 0ull;
        if (hi >= 0 && lo <= 63) {
          const int lc = max(lo, 0), hc = min(hi, 63);
          bm = (~0ull >> (63 - (hc - lc))) << lc;
        }
        m &= bm;
      }
      if (!qok) m = 0ull;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t w = (uint32_t)(m >> (32 * kb));
        asm("" : "+v"(w));
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = keep_if_bit(sc[kb][r], w, 8 * (r >> 2) + (r & 3), ninf);
      }
    }
    // Online softmax per 32-key half against the row's reference ref: weights 2^(x - ref).
    // Fast path: exponentiate without a row max and accept when every lane's 16 weights sum to
    // at most 2^16 (no weight above 2^16, nothing overflows).  Otherwise (a row's first allowed
    // key, or a score far above ref) take the half's row max; a row moves ref to it when it has
    // none yet or when the max exceeds ref by more than 2^8, and the weights are redone.  Then
    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16& u = sc[kb];
      uint32_t pk[8];
      float part = 0.f;
      auto exponentiate = [&]() {
        const float add = off - ref;
        float la = 0.f, lb = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2_fast(__builtin_fmaf(u[r], mul, add));
          const float p1 = exp2_fast(__builtin_fmaf(u[r + 1], mul, add));
          pk[r >> 1] = pack_bf16x2(p0, p1);
          // rounded weights, as the PV products use them
          if (r & 2) lb = add_bf16x2(pk[r >> 1], lb);
          else la = add_bf16x2(pk[r >> 1], la);
        }
        part = la + lb;
      };
      exponentiate();
      if (__builtin_amdgcn_ballot_w64(!has | !(part <= kTgFastWeightSum)) != 0ull) {
        float x0 = __builtin_fmaxf(__builtin_fmaxf(u[0], u[1]), u[2]);
        float x1 = __builtin_fmaxf(__builtin_fmaxf(u[3], u[4]), u[5]);
        x0 = __builtin_fmaxf(__builtin_fmaxf(x0, u[6]), u[7]);
        x1 = __builtin_fmaxf(__builtin_fmaxf(x1, u[8]), u[9]);
        x0 = __builtin_fmaxf(__builtin_fmaxf(x0, u[10]), u[11]);
        x1 = __builtin_fmaxf(__builtin_fmaxf(x1, u[12]), u[13]);
        x0 = __builtin_fmaxf(__builtin_fmaxf(x0, u[14]), __builtin_fmaxf(x1, u[15]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x0),
                                                         false, false);
        const float xm = __builtin_fmaf(
            __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), mul, off);
        const bool need = (xm != ninf) & (!has | (xm - ref > kRefSlack));
        if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
          const float nref = need ? xm : ref;
          const float alpha = has ? exp2_fast(ref - nref) : 1.f;
          ref = nref;
          has = has || need;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        exponentiate();
      }
      l_run += part;
#pragma unroll
      for (int gh = 0; gh < 2; ++gh) {
        const int g = 2 * kb + gh;
        const u32x4 bp = {pk[4 * gh], pk[4 * gh + 1], pk[4 * gh + 2], pk[4 * gh + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const unsigned char* vp = sv_ + voffs[db] + 16 * g * (2 * D);
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp + 8 * (2 * D)));
          const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
          o[db] = mfma_32x32x16(u32x4{w0[0], w0[1], w1[0], w1[1]}, bp, o[db]);
        }
      }
    }
  };

  // does tile t reach this wave's rows? (local tiles outside every row's window are skipped)
  auto reach = [&](int t) -> bool {
    if (!wave_rows) return false;
    if (t >= n_local) return true;
    const int kf = k_lo + t * kKeyTile, kl = kf + kKeyTile - 1;
    return !(kl < w_first - a.radius || kf > w_last + a.radius);
  };

  int st = 0;
  for (int t = 0; t < n_tiles; ++t) {
    if (t > 0) __syncthreads();
    const bool more = t + 1 < n_tiles;
    if (more) issue(st ^ 1, t + 1);
    if (more) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (reach(t)) tile(st, t);
    st ^= 1;
  }

  // epilogue: O = O^T / l, lse
  const float l_tot = l_run + __uint_as_float(__shfl_xor(__float_as_uint(l_run), 32));
  if (!qok) return;
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  uint16_t* orow = a.out + (bh * a.n + qpos) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = 32 * db + 8 * rq + 4 * hh;
      u32x2 w;
      w[0] = pack_bf16x2(o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv);
      w[1] = pack_bf16x2(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d) = w;
    }
  if (a.lse && hh == 0)
    a.lse[bh * a.n + qpos] = (l_tot > 0.f) ? (ref + __log2f(l_tot)) * kLn2 : neg_inf();
}

}  // namespace

hipError_t launch_tglobal_side(const TgArgs& a, const uint16_t* x, const float* gamma,
                               const uint16_t* wk, const uint16_t* wv, uint16_t* y,
                               hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const dim3 agrid((unsigned)(a.B * a.G));
  const int groups = a.dm / 8;  // 8-column groups of a row
  if (groups <= 64) hipLaunchKernelGGL(tg_aggregate_kernel<1>, agrid, dim3(64), 0, s, a, x, gamma, y);
  else if (groups <= 128) hipLaunchKernelGGL(tg_aggregate_kernel<2>, agrid, dim3(64), 0, s, a, x, gamma, y);
  else if (groups <= 256) hipLaunchKernelGGL(tg_aggregate_kernel<4>, agrid, dim3(64), 0, s, a, x, gamma, y);
  else hipLaunchKernelGGL(tg_aggregate_kernel<8>, agrid, dim3(64), 0, s, a, x, gamma, y);
  const long rows = (long)a.B * a.G;
  const dim3 grid((unsigned)((rows + kProjTile - 1) / kProjTile),
                  (unsigned)((a.H * a.D + kProjTile - 1) / kProjTile), 2);
  hipLaunchKernelGGL(tg_project_kernel, grid, dim3(64), 0, s, a, y, wk, wv);
  return hipGetLastError();
}

hipError_t launch_tglobal_attention(const TgArgs& a, const float* tab_local,
                                    const float* tab_side, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(tg_bias_kernel, dim3(4, a.H), dim3(256), 0, s, a, tab_local, tab_side);
  const long grid = (long)a.B * a.H * ((a.n + 127) / 128);
  if (a.D == 64)
    hipLaunchKernelGGL(tg_attn_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else if (a.D == 128)
    hipLaunchKernelGGL(tg_attn_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace longattn
