// bf16 backward pass of the window / dilation / global-token and block-layout patterns on gfx950
// matrix cores.
//
// With the forward's log-normaliser of every query row (kept in log2 units, lse2), the softmax
// weights of an edge are recomputed directly, P = 2^(c2 s - lse2), c2 = scale * log2(e), so no
// online softmax is needed.  For an edge (query i, key j), with Drow_i = dO_i . O_i:
//   dP = dO_i . v_j,  dS = P (dP - Drow_i),
//   dQ_i += scale * dS k_j,  dK_j += scale * dS q_i,  dV_j += P dO_i.
// Every gradient row has one owner, so there are no atomics.  Two launches of one kernel
// template (then one combine for the global tokens):
//   dQ kind:   a wave owns 32 query rows (its Q and dO rows are MFMA B operands held in
//              registers) and streams 64-key tiles of K and V through LDS, like the forward pass;
//              it also computes every row's Drow and lse2 once and stores them for the next;
//   dK/dV kind: a wave owns 32 key rows (K and V rows in registers) and streams 64-row tiles of
//              Q and dO through LDS, with each streamed row's lse2 and Drow.
// In both, the streamed rows s of owner row o satisfy o - WL <= s <= o + WR in the residue
// subsequence of the dilation (the window splits into independent undilated windows on the
// residue classes; Longformer hub page, section 2): (WL, WR) = (win_left, win_right) for the dQ
// kind and (win_right, win_left) for the dK/dV kind, because key j is in the window of query i
// exactly when i is in the mirrored window of j.
//
// Global tokens (Longformer hub page, section 2; Big Bird reading notes, section 3.2.3): window
// tiles drop the streamed rows that are global tokens (their edges go through the global paths,
// each edge counted once, as in the forward pass); window workgroups then walk the global rows
// as gathered tiles (global keys for dQ, global query rows for dK/dV).  The owners that are global
// tokens (global query rows for dQ, global keys for dK/dV) get their own workgroups, one per
// (batch, head, 128 global rows, 512-row chunk), dispatched after the window workgroups so that
// they fill the last round, which stream every position of the chunk and write fp32 partial
// sums; a combine kernel adds the chunks and overwrites those rows.
//
// Block layouts (Big Bird reading notes, sections 3.2.2 and 3.3): a dQ workgroup owns a query
// block and streams its listed key blocks; a dK/dV workgroup owns a key block and streams the
// query blocks whose layout rows list it (found by scanning the layout).  As in the forward pass,
// a global key inside a listed block is attended through the block.
//
// Wave-level math (32x32x16 bf16 MFMA, fp32 accumulate).  Scores come out as C[streamed row]
// [owner row]: every lane holds one owner row (its column) against 32 streamed rows.  The
// gradient sums are kept transposed, G^T[d][owner] += X^T[d][streamed] C[streamed][owner], so
// the C blocks (P or dS, rounded to bf16) serve directly as B operands and X^T is read from LDS
// with the transposing 64-bit read.  Streamed matrices read both ways use the transposing
// layout's swizzle.

#include <type_traits>

#include <hip/hip_ext.h>

#include "attn_args.h"
#include "mfma_util.h"

#ifndef BWD_DV_WAVES_128
#define BWD_DV_WAVES_128 2
#endif
#ifndef BWD_SPLIT_DKV_MASK
#define BWD_SPLIT_DKV_MASK 2  // bit 0: d = 64, bit 1: d = 128
#endif

namespace longattn {
namespace {

using namespace mfma;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBwdPadWords = 64;  // staged key-padding and global-row bits: 4096 positions
constexpr int kBwdMaxBlocks = 1024;  // layout mode: listed (or listing) blocks per workgroup

template <int D>
struct BwdSmem {
  __attribute__((aligned(1024))) unsigned char stage_a[2][kKeyTile * D * 2];  // K or Q
  __attribute__((aligned(1024))) unsigned char stage_b[2][kKeyTile * D * 2];  // V or dO
  __attribute__((aligned(16))) float row_l[2][kKeyTile];  // dK/dV: lse2 of the streamed rows
  __attribute__((aligned(16))) float row_d[2][kKeyTile];  // dK/dV: Drow of the streamed rows
  __attribute__((aligned(16))) int g_pos[kGlobalCap];     // global rows: positions
  unsigned long long g_valid[kGlobalCap / 64];             // global rows: usable bits
  unsigned long long g_bits[kBwdPadWords];                 // global rows among window rows
  unsigned long long pad_bits[kBwdPadWords];               // dQ: key padding of window keys
  int lay_list[kBwdMaxBlocks];  // layout mode: streamed blocks (dQ: listed key blocks of the
                                // query block; dK/dV: query blocks that list the key block)
  int lay_cnt;
};

struct STile {
  int gathered;  // 0: row r at position base + kst * r; 1: row r is global row base + r
  int base;
  int count;     // rows >= count do not exist
  int ks0;       // window tiles: residue-subsequence index of row 0
  int lt;        // window tiles: index of the tile within the workgroup's streamed range
};

// Occupancy: the dQ kind is held to 168 VGPRs at d = 64 (three waves per SIMD) and 256 at
// d = 128 (two); one wave per SIMD more than a few extra registers would leave (measured: the dQ
// kernel 15% faster on dilated_16k, 35% on swa512_causal_32k).  Working on the streamed tile in
// 32-row halves keeps it within those bounds without spilling.  The dK/dV kind needs its
// registers (capping it spills).
template <int D, int KIND, int NW, int MODE_MAIN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(
    (KIND == kBwdDQ || KIND == kBwdDK) ? (D == 64 ? 3 : 2)
                                       : (KIND == kBwdDV ? (D == 64 ? 4 : BWD_DV_WAVES_128) : 1))))
void attn_bwd_kernel(FwdArgs args, BwdArgs gargs) {
  __shared__ BwdSmem<D> sm;
  const FwdCore a = args;
  const BwdArgs gp = gargs;
  const int total = gridDim.x;
  const int n_glob_wg = a.grid_rows;
  const int n_main_wg = total - n_glob_wg;
  // the window workgroups first (consecutive indices on one XCD), then the global owners
  const int gi = (int)blockIdx.x >= n_main_wg ? (int)blockIdx.x - n_main_wg : -1;
  const int mi = gi < 0 ? xcd_remap(blockIdx.x, n_main_wg) : 0;

  int main_b = 0, main_h = 0, main_dl = 1, main_r = 0;
  if (gi < 0) {
    main_b = mi / a.tiles_per_b;
    int r = mi - main_b * a.tiles_per_b;
    if (a.head_tiles > 0) {
      main_h = r / a.head_tiles;
      r -= main_h * a.head_tiles;
      main_dl = a.uniform_dil > 0 ? a.uniform_dil : args.dil[main_h];
    } else {
      int lo = 0, hi = a.H - 1;  // last head with tile_off[h] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (args.tile_off[mid] <= r) lo = mid; else hi = mid - 1;
      }
      main_h = lo;
      r -= args.tile_off[main_h];
      main_dl = args.dil[main_h];
    }
    main_r = r;
  }

  auto body = [&](auto mode_c, const int wg) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool DQ = KIND == kBwdDQ;
    constexpr bool ACC0 = KIND != kBwdDV;                       // dQ^T or dK^T
    constexpr bool ACC1 = KIND == kBwdDKV || KIND == kBwdDV;    // dV^T
    constexpr bool NEED_DP = KIND != kBwdDV;                    // dP (for dS)
    constexpr int NT = NW * 64, RW = 32, QT = NW * RW;
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int KS = D / 16;         // MFMA k-steps over the head dim
    constexpr int DB = D / 32;         // 32-row blocks of a transposed gradient
    constexpr int NLOAD = 2 * CH;      // 1 KB direct-load blocks per tile (matrix A, then B)
    constexpr int LPW = NLOAD / NW;
    constexpr int RPB = 64 / CH;       // rows per 1 KB block
    constexpr bool kGathered = MODE != kGlobalRows;  // main workgroups also walk the global rows
    constexpr int GREG = kGlobalCap / NT;            // global rows staged per thread
    static_assert(NLOAD % NW == 0 && CH % LPW == 0, "each wave loads whole blocks of one matrix");
    static_assert(kGlobalCap % NT == 0, "whole rounds of global rows when staging");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qj = lane & 31, hh = lane >> 5;
    const int WL = DQ ? a.wl : a.wr, WR = DQ ? a.wr : a.wl;

    // ------------------------------------------------------------------ work decomposition
    int b = 0, h = 0, dl = 1, p = 0, np = a.n, o0 = 0, ck = 0, rg = 0;
    if constexpr (MODE == kGlobalRows) {
      const int rgs = (a.g + QT - 1) / QT;
      if (a.rows_by_xcd) {
        // as in the forward: XCD x (blockIdx.x % 8) ran the main work of (batch, head) pairs
        // x*hpx .. x*hpx + hpx - 1 in order; its global-owner workgroups take those pairs, the
        // most recent first, chunks from the last rows down
        const int per = rgs * a.chunks;
        const int hpx = (a.B * a.H) >> 3;
        const int s = wg >> 3, i = s / per, u = s - i * per;
        const int bhx = (wg & 7) * hpx + hpx - 1 - i;
        b = bhx / a.H;
        h = bhx - b * a.H;
        rg = u / a.chunks;
        ck = a.chunks - 1 - (u - rg * a.chunks);
      } else {
        int x = wg;
        ck = x % a.chunks;
        x /= a.chunks;
        rg = x % rgs;
        x /= rgs;
        h = x % a.H;
        b = x / a.H;
      }
    } else {
      (void)wg;
      b = main_b;
      h = main_h;
      dl = main_dl;
      int r = main_r;
      if constexpr (MODE == kBand) {
        for (;;) {  // residue class p holds ceil((n - p) / dl) positions
          const int n_p = (a.n - p + dl - 1) / dl;
          const int t_p = (n_p + QT - 1) / QT;
          if (r < t_p) { np = n_p; break; }
          r -= t_p;
          ++p;
        }
      }
      o0 = r * QT;  // kLayout: block r (QT == block)
    }
    const int kst = (MODE == kBand) ? min(dl, a.n) : 1;
    const long bh = (long)b * a.H + h;
    const uint16_t* dOb = static_cast<const uint16_t*>(gp.dout) + bh * a.n * D;
    const uint16_t* SA = (DQ ? a.k : a.q) + bh * a.n * D;   // streamed matrix A
    const uint16_t* SB = DQ ? a.v + bh * a.n * D : dOb;     // streamed matrix B
    const uint16_t* OA = (DQ ? a.q : a.k) + bh * a.n * D;   // owner matrix A
    const uint16_t* OB = DQ ? dOb : a.v + bh * a.n * D;     // owner matrix B
    const float* l2b = gp.lse2 + bh * a.n;
    const float* drb = gp.drow + bh * a.n;
    const uint8_t* pad = a.kpad ? a.kpad + (long)b * a.n : nullptr;
    const int* gb = a.gidx ? a.gidx + (long)b * a.g : nullptr;

    // ------------------------------------------------------------------ owner row of this lane
    int opos = -1, osub = 0;
    {
      const int orow = wave * RW + qj;
      if constexpr (MODE == kBand) {
        osub = o0 + orow;
        if (osub < np) opos = p + dl * osub;
      } else if constexpr (MODE == kLayout) {
        osub = o0 + orow;
        opos = osub;
      } else {
        const int c = rg * QT + orow;
        if (c < a.g) {
          const int x = gb[c];
          if (x >= 0 && x < a.n) opos = x;
        }
      }
    }
    // ------------------------------------------------------------------ streamed tiles
    int n_local = 0, s_lo = 0, s_hi = -1;
    constexpr int TPB = QT / kKeyTile;  // layout mode: key tiles per block (QT rows)
    if constexpr (MODE == kLayout) {
      // dQ: the valid key blocks listed for this query block; dK/dV: the query blocks whose
      // layout row lists this key block, in ascending order (compacted by wave 0)
      const int nb = a.n / a.block;
      const int me = o0 / a.block;
      if (wave == 0) {
        int base = 0;
        if constexpr (DQ) {
          const int* row = a.layout + ((long)h * nb + me) * a.max_kb;
          for (int e0 = 0; e0 < a.max_kb; e0 += 64) {
            const int e = e0 + lane;
            int id = (e < a.max_kb) ? row[e] : -1;
            if (id >= nb) id = -1;  // out-of-range ids are ignored rather than read
            const unsigned long long m = __ballot(id >= 0);
            if (id >= 0) sm.lay_list[base + __popcll(m & ((1ull << lane) - 1ull))] = id;
            base += __popcll(m);
          }
        } else {
          for (int q0b = 0; q0b < nb; q0b += 64) {
            const int qb = q0b + lane;
            bool lists = false;
            if (qb < nb) {
              const int* row = a.layout + ((long)h * nb + qb) * a.max_kb;
              for (int e = 0; e < a.max_kb; ++e) lists = lists | (row[e] == me);
            }
            const unsigned long long m = __ballot(lists);
            if (lists) sm.lay_list[base + __popcll(m & ((1ull << lane) - 1ull))] = qb;
            base += __popcll(m);
          }
        }
        if (lane == 0) sm.lay_cnt = base;
      }
      __syncthreads();
      n_local = sm.lay_cnt * TPB;
    } else if constexpr (MODE == kBand) {
      if (a.band_on) {
        const int o_last = min(o0 + QT, np) - 1;
        s_lo = max(0, o0 - WL);
        s_hi = min(np - 1, o_last + WR);
        n_local = (s_hi >= s_lo) ? (s_hi - s_lo + kKeyTile) / kKeyTile : 0;
      }
    } else {
      const int c0 = ck * a.chunk_keys;
      const int c1 = min(a.n, c0 + a.chunk_keys);
      n_local = (c1 > c0) ? (c1 - c0 + kKeyTile - 1) / kKeyTile : 0;
      s_lo = c0;
      s_hi = c1 - 1;
    }
    const int n_gtiles = (kGathered && a.g > 0) ? (a.g + kKeyTile - 1) / kKeyTile : 0;
    const int n_tiles = n_local + n_gtiles;
    // At head dim 64 the window tiles are streamed in a rotated order: step t takes the tile
    // whose residue-subsequence index, (s_lo / 64) + lt, is congruent to t modulo n_local, so
    // neighbouring owner tiles read the same streamed tile at the same step and the re-reads hit
    // the XCD's L2 (the same walk as the forward pass; the sums do not depend on the order).
    int rot = 0;
    if constexpr (MODE == kBand && D == 64) {
      if (n_local > 0) rot = (n_local - (s_lo / kKeyTile) % n_local) % n_local;
    }

    auto tile_of = [&](int t) -> STile {
      STile T;
      T.ks0 = 0;
      T.lt = 0;
      if (t >= n_local) {
        T.gathered = 1;
        T.base = (t - n_local) * kKeyTile;
        T.count = min(kKeyTile, a.g - T.base);
      } else if constexpr (MODE == kBand) {
        T.gathered = 0;
        if constexpr (D == 64) T.lt = t + rot < n_local ? t + rot : t + rot - n_local;
        else T.lt = t;
        T.ks0 = s_lo + T.lt * kKeyTile;
        T.base = p + dl * T.ks0;
        T.count = min(kKeyTile, np - T.ks0);
      } else if constexpr (MODE == kLayout) {
        T.gathered = 0;
        T.base = sm.lay_list[t / TPB] * a.block + (t % TPB) * kKeyTile;
        T.count = kKeyTile;
      } else {
        T.gathered = 0;
        T.base = s_lo + t * kKeyTile;
        T.count = min(kKeyTile, s_hi + 1 - T.base);
      }
      return T;
    };

    // ------------------------------------------------------------------ tile loading
    // Waves 0-1 move matrix A's 1 KB blocks, waves 2-3 matrix B's (block `sub` holds rows
    // RPB*sub .. +RPB-1; lane l moves row RPB*sub + l/CH, chunk l%CH, to its swizzled slot).
    // For dK/dV, wave 0 also moves the tile rows' lse2 and wave 1 their Drow (4 bytes a lane).
    const int mat = (wave * LPW) / CH;
    const int sub0 = (wave * LPW) % CH;
    const bool vlayout = (mat == 0) || !DQ;  // matrices read transposed use that layout
    auto ld_row = [&](int j) -> int { return (sub0 + j) * RPB + lane / CH; };
    auto ld_col = [&](int j) -> int {
      const int row = ld_row(j);
      return 8 * ((lane % CH) ^ (vlayout ? swz_v<D>(row) : swz_k<D>(row)));
    };
    uint32_t voff[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      voff[j] = (uint32_t)(min((long)ld_row(j) * kst, (long)a.n) * D + ld_col(j)) * 2u;
    const uint16_t* msrc = (mat == 0) ? SA : SB;
    const bool row_wave = !DQ && wave < 2;
    const float* row_src = wave == 0 ? l2b : drb;
    auto issue = [&](int si, const STile& T) {
      unsigned char* stg = mat == 0 ? sm.stage_a[si] : sm.stage_b[si];
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stg + sub0 * 1024));
      if (kGathered && T.gathered) {
        const u32x4 rs = buf_rsrc(msrc, (uint32_t)a.n * D * 2u);
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
          const int pos = sm.g_pos[T.base + min(ld_row(j), T.count - 1)];
          lds_dma16(rs, (uint32_t)(pos * D + ld_col(j)) * 2u, dst + 1024 * j);
        }
      } else {
        const u32x4 rs = buf_rsrc(msrc + (long)T.base * D, (uint32_t)(a.n - T.base) * D * 2u);
#pragma unroll
        for (int j = 0; j < LPW; ++j) lds_dma16(rs, voff[j], dst + 1024 * j);
      }
      if (row_wave) {
        float* rdst = wave == 0 ? sm.row_l[si] : sm.row_d[si];
        const uint32_t dw = __builtin_amdgcn_readfirstlane(lds_addr(rdst));
        uint32_t off;
        if (kGathered && T.gathered)
          off = (uint32_t)sm.g_pos[T.base + min(lane, T.count - 1)] * 4u;
        else
          off = lane < T.count ? (uint32_t)(T.base + kst * lane) * 4u : (uint32_t)a.n * 4u;
        lds_dma4(buf_rsrc(row_src, (uint32_t)a.n * 4u), off, dw);
      }
    };

    // Global rows first (positions feed the gathered tiles and the window-tile exclusion), then
    // the first window tile, the owner fragments and the staging.
    int gx[GREG];
#pragma unroll
    for (int i = 0; i < GREG; ++i) {
      const int c = tid + NT * i;
      gx[i] = (kGathered && n_gtiles > 0 && c < a.g) ? gb[c] : a.n;
    }
    if (n_local > 0) issue(0, tile_of(0));

    // Owner fragments (B operands): lane (qj, hh) holds d = 16ks + 8hh .. +7 of its owner row.
    const float c2 = a.scale_log2;
    u32x4 fa[KS], fb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      fa[s] = u32x4{0, 0, 0, 0};
      fb[s] = u32x4{0, 0, 0, 0};
      if (opos >= 0) {
        fa[s] = *reinterpret_cast<const u32x4*>(OA + (long)opos * D + 16 * s + 8 * hh);
        if (NEED_DP || DQ)
          fb[s] = *reinterpret_cast<const u32x4*>(OB + (long)opos * D + 16 * s + 8 * hh);
      }
    }
    // dQ: the owner query's lse2 (lse in log2 units; 0 for an empty row, whose edges are all
    // masked) and Drow = dO . O (this lane's half of the head dim, then the partner lane's);
    // the main workgroups own every row once and leave both for the dK/dV kernel.
    float o_l2 = 0.f, o_dr = 0.f;
    bool own_ok = opos >= 0;  // dK/dV: the owner key exists and is not padded
    if constexpr (DQ) {
      float lse = 0.f;
      u32x4 of[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        of[s] = u32x4{0, 0, 0, 0};
        if (opos >= 0)
          of[s] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(gp.out) +
                                                  (bh * a.n + opos) * D + 16 * s + 8 * hh);
      }
      if (opos >= 0) lse = a.lse[bh * a.n + opos];
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part = __builtin_fmaf(__uint_as_float(of[s][e] << 16), __uint_as_float(fb[s][e] << 16), part);
          part = __builtin_fmaf(__uint_as_float(of[s][e] & 0xffff0000u),
                                __uint_as_float(fb[s][e] & 0xffff0000u), part);
        }
      o_dr = part + __shfl_xor(part, 32);
      o_l2 = lse == -__builtin_inff() ? 0.f : lse * kLog2e;
      if (MODE != kGlobalRows && opos >= 0 && hh == 0) {
        gp.drow[bh * a.n + opos] = o_dr;
        gp.lse2[bh * a.n + opos] = o_l2;
      }
    } else {
      if (own_ok && pad) own_ok = pad[opos] == 0;
    }

    // ------------------------------------------------------------------ staging in LDS
    // Usable global rows: dQ streams global keys (in range, not padded); dK/dV streams global
    // query rows (in range).  Window tiles drop them (g_bits over the window range when it fits,
    // else a search of the sorted positions).
    const bool gbits_staged = MODE == kBand && n_gtiles > 0 && n_local <= kBwdPadWords;
    if constexpr (kGathered) {
      if (n_gtiles > 0) {
        if (gbits_staged) {
          for (int w = tid; w < n_local; w += NT) sm.g_bits[w] = 0ull;
          __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < GREG; ++i) {
          const int c = tid + NT * i;
          const int x = gx[i];
          bool ok = c < a.g && x >= 0 && x < a.n;
          if constexpr (DQ) {
            if (ok && pad) ok = pad[x] == 0;
          }
          const int pos = min(max(x, 0), a.n);
          if constexpr (DQ && MODE == kLayout) {
            // a global key inside one of the listed blocks is attended through the block
            const int blk = pos / a.block;
            for (int e = 0; e < sm.lay_cnt; ++e) ok = ok && (sm.lay_list[e] != blk);
          }
          if constexpr (MODE == kBand) {
            const int rel = pos - p;
            if (gbits_staged && ok && rel >= 0 && rel % dl == 0) {
              const int j = rel / dl - s_lo;
              if (j >= 0 && j < kKeyTile * n_local) atomicOr(&sm.g_bits[j >> 6], 1ull << (j & 63));
            }
          }
          sm.g_pos[c] = pos;
          const unsigned long long vm = __ballot(ok);
          if (lane == 0) sm.g_valid[c >> 6] = vm;
        }
      }
    }
    // dQ: key padding of the reachable window positions as bits, when they fit.
    int pad_lo = 0;
    bool pad_staged = false;
    if (DQ && pad && n_local > 0) {
      long lo, hi;
      if constexpr (MODE == kBand) {
        lo = p + (long)dl * s_lo;
        hi = min((long)a.n - 1, p + (long)dl * (s_lo + (long)kKeyTile * n_local - 1));
      } else if constexpr (MODE == kLayout) {
        lo = 0;
        hi = a.n - 1;
      } else {
        lo = s_lo;
        hi = s_hi;
      }
      lo &= ~63L;
      const long words = ((hi - lo) >> 6) + 1;
      pad_staged = words <= kBwdPadWords;
      pad_lo = (int)lo;
      if (pad_staged) {
        for (int w = wave; w < (int)words; w += NW) {
          const int pos = pad_lo + 64 * w + lane;
          const unsigned long long m = __ballot(pos < a.n && pad[pos] == 0);
          if (lane == 0) sm.pad_bits[w] = m;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      asm volatile("" : : "v"(fa[s]));
      if constexpr (NEED_DP) asm volatile("" : : "v"(fb[s]));
    }
    __syncthreads();
    if (n_local == 0 && n_tiles > 0) issue(0, tile_of(0));

    // bits of the global rows among the rows of window tile t (they are dropped there)
    auto global_rows = [&](const STile& T, int t) -> unsigned long long {
      if (n_gtiles == 0) return 0ull;
      if (gbits_staged) return sm.g_bits[t];
      const bool in = lane < T.count;
      const int pos = in ? T.base + kst * lane : 0;
      int c = -1;  // last global row with position <= pos (positions ascend)
#pragma unroll
      for (int step = kGlobalCap; step > 0; step >>= 1)
        if (c + step < a.g && sm.g_pos[c + step] <= pos) c += step;
      const bool hit = in && c >= 0 && sm.g_pos[c] == pos && ((sm.g_valid[c >> 6] >> (c & 63)) & 1ull);
      return __ballot(hit);
    };
    // usable streamed rows of a local tile: they exist and (dQ) the key is not padded
    auto local_valid = [&](const STile& T) -> unsigned long long {
      const unsigned long long cnt = T.count >= 64 ? ~0ull : ((1ull << T.count) - 1ull);
      if (!DQ || !pad) return cnt;
      const bool in = lane < T.count;
      const long pos = in ? (long)T.base + (long)kst * lane : 0;
      bool ok;
      if (pad_staged) {
        const int rel = in ? (int)(pos - pad_lo) : 0;
        ok = in && ((sm.pad_bits[rel >> 6] >> (rel & 63)) & 1ull);
      } else {
        ok = in && pad[pos] == 0;
      }
      return __ballot(ok);
    };

    // ------------------------------------------------------------------ per-lane LDS offsets
    // Row-major A operand (streamed row 32kb + qj, k-step ks): logical chunk 2ks + hh.
    const int swa = swz_v<D>(qj);
    const int swb = DQ ? swz_k<D>(qj) : swz_v<D>(qj);
    int koa[KS], kob[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      koa[ks] = qj * (2 * D) + (((2 * ks + hh) ^ swa) * 16);
      kob[ks] = qj * (2 * D) + (((2 * ks + hh) ^ swb) * 16);
    }
    // Transposed A operand for 16-row group t, d block db, half r (as in the forward pass).
    const int vi = lane & 15, vg = lane >> 4;
    const int vrow0 = 4 * hh + (vi >> 2);
    const int vsw = swz_v<D>(vrow0);
    int toffs[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 4 * db + 2 * (vg & 1) + ((vi & 3) >> 1);
      toffs[db] = vrow0 * (2 * D) + ((chunk ^ vsw) * 16) + 8 * (vi & 1);
    }
    auto read_t = [&](const unsigned char* stg, int grp, int db) -> u32x4 {
      const unsigned char* vp = stg + toffs[db] + 16 * grp * (2 * D);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp + 8 * (2 * D)));
      const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      return u32x4{w0[0], w0[1], w1[0], w1[1]};
    };

    // ------------------------------------------------------------------ accumulators
    // acc0: dQ^T (dQ kind) or dK^T; acc1: dV^T.  Register r of block db is d = 32db + 8(r/4) +
    // 4hh + r%4 of the lane's owner row.
    f32x16 acc0[DB], acc1[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc0[db][r] = 0.f;
        acc1[db][r] = 0.f;
      }

    const int w_first = o0 + wave * RW;
    const int w_last = (MODE == kBand) ? min(w_first + RW - 1, np - 1) : w_first + RW - 1;
    bool wave_rows;
    if constexpr (MODE == kBand) wave_rows = w_first < np;
    else if constexpr (MODE == kLayout) wave_rows = true;
    else wave_rows = (rg * QT + wave * RW) < a.g;

    auto reach = [&](const STile& T, bool& need_band) -> bool {
      need_band = false;
      if (!wave_rows) return false;
      if constexpr (MODE == kBand) {
        if (!T.gathered) {
          const int kf = T.ks0, kl = T.ks0 + kKeyTile - 1;
          if (kl < w_first - WL || kf > w_last + WR) return false;
          need_band = !(kf >= w_last - WL && kl <= w_first + WR);
        }
      }
      return true;
    };

    // ------------------------------------------------------------------ one tile
    auto compute = [&](int si, const STile& T, unsigned long long vmask, bool need_band) {
      const unsigned char* sa = sm.stage_a[si];
      const unsigned char* sb = sm.stage_b[si];
      // per 32-row half kb of the streamed tile: raw scores and dP (both C[streamed][owner]),
      // masks, P and dS, and the accumulation
      const bool masked = need_band || vmask != ~0ull ||
                          (!DQ && __builtin_amdgcn_ballot_w64(!own_ok) != 0ull);
      unsigned long long m = vmask >> (4 * hh);
      if (need_band) {
        const int lo = osub - WL - T.ks0 - 4 * hh;
        const int hi = osub + WR - T.ks0 - 4 * hh;
        unsigned long long bm = 0ull;
        if (hi >= 0 && lo <= 63) {
          const int lc = max(lo, 0), hc = min(hi, 63);
          bm = (~0ull >> (63 - (hc - lc))) << lc;
        }
        m &= bm;
      }
      if (!own_ok && !DQ) m = 0ull;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = 0.f;
          dp[r] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 xa = *reinterpret_cast<const u32x4*>(sa + koa[ks] + kb * 32 * (2 * D));
          sc = mfma_32x32x16(xa, fa[ks], sc);
        }
        if constexpr (NEED_DP) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u32x4 xb = *reinterpret_cast<const u32x4*>(sb + kob[ks] + kb * 32 * (2 * D));
            dp = mfma_32x32x16(xb, fb[ks], dp);
          }
        }
        if (masked) {
          const float ninf = neg_inf();
          uint32_t w = (uint32_t)(m >> (32 * kb));
          asm("" : "+v"(w));
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[r] = keep_if_bit(sc[r], w, 8 * (r >> 2) + (r & 3), ninf);
        }
        uint32_t pk[8], dk[8];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float l4[4], d4[4];
          if constexpr (DQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              l4[e] = o_l2;
              d4[e] = o_dr;
            }
          } else {
            const int row = 32 * kb + 8 * q4 + 4 * hh;
            const float4 L = *reinterpret_cast<const float4*>(&sm.row_l[si][row]);
            const float4 R = *reinterpret_cast<const float4*>(&sm.row_d[si][row]);
            l4[0] = L.x; l4[1] = L.y; l4[2] = L.z; l4[3] = L.w;
            d4[0] = R.x; d4[1] = R.y; d4[2] = R.z; d4[3] = R.w;
          }
          float pe[4], de[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            pe[e] = exp2_fast(__builtin_fmaf(sc[r], c2, -l4[e]));
            de[e] = pe[e] * (dp[r] - d4[e]);
          }
          pk[2 * q4] = pack_bf16x2(pe[0], pe[1]);
          pk[2 * q4 + 1] = pack_bf16x2(pe[2], pe[3]);
          dk[2 * q4] = pack_bf16x2(de[0], de[1]);
          dk[2 * q4 + 1] = pack_bf16x2(de[2], de[3]);
        }
        // G^T += X^T C over the 16-row groups 2kb, 2kb+1
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
          const int grp = 2 * kb + gh;
          const u32x4 bds = {dk[4 * gh], dk[4 * gh + 1], dk[4 * gh + 2], dk[4 * gh + 3]};
          const u32x4 bp = {pk[4 * gh], pk[4 * gh + 1], pk[4 * gh + 2], pk[4 * gh + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            if constexpr (ACC0) acc0[db] = mfma_32x32x16(read_t(sa, grp, db), bds, acc0[db]);
            if constexpr (ACC1) acc1[db] = mfma_32x32x16(read_t(sb, grp, db), bp, acc1[db]);
          }
        }
      }
    };

    // ------------------------------------------------------------------ tile loop
    // Two stages per matrix; step t refills the stage of tile t-1 with tile t+1, waits for this
    // wave's loads of tile t (tile t+1's stay in flight), then a barrier publishes tile t.
    if (n_tiles > 0) {
      int st = 0;
      for (int t = 0; t < n_tiles; ++t) {
        if (t > 0) __syncthreads();
        const bool more = t + 1 < n_tiles;
        if (more) issue(st ^ 1, tile_of(t + 1));
        if (more) {
          if (row_wave) wait_vmcnt<LPW + 1>();
          else wait_vmcnt<LPW>();
        } else {
          wait_vmcnt<0>();
        }
        __syncthreads();
        const STile T = tile_of(t);
        bool need_band = false;
        if (reach(T, need_band)) {
          // window tiles drop the global rows (they go through the global paths); listed layout
          // blocks keep global keys (dQ: the global column skips them) but drop global query
          // rows (dK/dV: those rows are streamed from the global list)
          unsigned long long vmask;
          if constexpr (MODE == kBand)
            vmask = T.gathered ? sm.g_valid[T.base >> 6] : local_valid(T) & ~global_rows(T, T.lt);
          else if constexpr (MODE == kLayout)
            vmask = T.gathered ? sm.g_valid[T.base >> 6]
                               : (DQ ? local_valid(T) : local_valid(T) & ~global_rows(T, T.lt));
          else
            vmask = local_valid(T);
          compute(st, T, vmask, need_band);
        }
        st ^= 1;
      }
    }

    // ------------------------------------------------------------------ epilogue
    if (opos < 0) return;
    const float scale = a.scale;
    if constexpr (MODE == kGlobalRows) {
      // fp32 partial sums (unscaled); the combine adds the chunks
      const int c = rg * QT + wave * RW + qj;
      const long slot = (bh * a.g + c) * a.chunks + ck;
      float* po = a.part + slot * (DQ ? D : 2 * D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + 4 * hh;
          if constexpr (ACC0)
            *reinterpret_cast<float4*>(po + d) =
                make_float4(acc0[db][4 * rq], acc0[db][4 * rq + 1], acc0[db][4 * rq + 2],
                            acc0[db][4 * rq + 3]);
          if constexpr (ACC1)
            *reinterpret_cast<float4*>(po + D + d) =
                make_float4(acc1[db][4 * rq], acc1[db][4 * rq + 1], acc1[db][4 * rq + 2],
                            acc1[db][4 * rq + 3]);
        }
    } else {
      uint16_t* g0 = static_cast<uint16_t*>(DQ ? gp.dq : gp.dk) + (bh * a.n + opos) * D;
      uint16_t* g1 = static_cast<uint16_t*>(gp.dv) + (bh * a.n + opos) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + 4 * hh;
          if constexpr (ACC0) {
            u32x2 w;
            w[0] = pack_bf16x2(acc0[db][4 * rq] * scale, acc0[db][4 * rq + 1] * scale);
            w[1] = pack_bf16x2(acc0[db][4 * rq + 2] * scale, acc0[db][4 * rq + 3] * scale);
            *reinterpret_cast<u32x2*>(g0 + d) = w;
          }
          if constexpr (ACC1) {
            u32x2 v;
            v[0] = pack_bf16x2(acc1[db][4 * rq], acc1[db][4 * rq + 1]);
            v[1] = pack_bf16x2(acc1[db][4 * rq + 2], acc1[db][4 * rq + 3]);
            *reinterpret_cast<u32x2*>(g1 + d) = v;
          }
        }
    }
  };
  if (gi >= 0) body(std::integral_constant<int, kGlobalRows>{}, gi);
  else body(std::integral_constant<int, MODE_MAIN>{}, mi);
}

// Adds the chunk partials of every global token and writes its dQ row (the global query row)
// and its dK and dV rows (the global key).  A workgroup of 192 threads takes 256 / D global
// tokens; thread t sums the column quad of one of the three that it owns over the chunks.
template <int D>
__global__ __launch_bounds__(192) void bwd_global_combine_kernel(FwdArgs args, BwdArgs gp) {
  constexpr int QPR = D / 4;           // column quads per row
  constexpr int TPR = 3 * QPR;         // threads per global token
  constexpr int RPW = 192 / TPR;       // global tokens per workgroup
  static_assert(RPW * TPR == 192, "whole tokens per workgroup");
  const FwdCore a = args;
  const int t = threadIdx.x;
  const long rows = (long)a.B * a.H * a.g;
  const long row = (long)blockIdx.x * RPW + t / TPR;
  if (row >= rows) return;  // no barrier follows
  const long bh = row / a.g;
  const int c = (int)(row - bh * a.g);
  const int b = (int)(bh / a.H);
  const int pos = a.gidx[(long)b * a.g + c];
  if (pos < 0 || pos >= a.n) return;
  const int which = (t % TPR) / QPR, col = 4 * (t % QPR);  // 0: dQ, 1: dK, 2: dV
  const long slots = (long)a.B * a.H * a.g * a.chunks;
  const long slot0 = (bh * a.g + c) * a.chunks;
  const float* po = which == 0 ? a.part + slot0 * D + col
                               : a.part + slots * D + slot0 * 2 * D + (which - 1) * D + col;
  const long stride = which == 0 ? D : 2 * D;
  // the loads of sixteen chunks go out together; the sums keep the chunk order
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 16
  for (int k = 0; k < a.chunks; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(po + k * stride);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  const float f = which == 2 ? 1.f : a.scale;
  u32x2 w;
  w[0] = pack_bf16x2(which == 2 ? s.x : s.x * f, which == 2 ? s.y : s.y * f);
  w[1] = pack_bf16x2(which == 2 ? s.z : s.z * f, which == 2 ? s.w : s.w * f);
  uint16_t* dst = static_cast<uint16_t*>(which == 0 ? gp.dq : which == 1 ? gp.dk : gp.dv) +
                  (bh * a.n + pos) * D + col;
  *reinterpret_cast<u32x2*>(dst) = w;
}

// dK and dV as two passes (each recomputes the scores; the dK pass also dP) where the fused
// dK/dV kind needs more registers than two waves per SIMD allow.
template <int D>
constexpr bool kBwdSplitDKV = BWD_SPLIT_DKV_MASK & (D / 64);

template <int D, int NW, int MODE>
hipError_t launch_bwd_d(const FwdArgs& a, const BwdArgs& g, long grid, hipStream_t s,
                        const LaunchEvents* ev) {
  auto launch = [&](hipEvent_t start, hipEvent_t stop, auto kernel, dim3 gr, dim3 bl,
                    auto... xs) {
    if (start || stop)
      hipExtLaunchKernelGGL(kernel, gr, bl, 0, s, start, stop, 0, xs...);
    else
      hipLaunchKernelGGL(kernel, gr, bl, 0, s, xs...);
  };
  auto timed = [&](int i, auto kernel, dim3 gr, dim3 bl, auto... xs) {
    launch(ev ? ev[i].start : nullptr, ev ? ev[i].stop : nullptr, kernel, gr, bl, xs...);
  };
  timed(0, attn_bwd_kernel<D, kBwdDQ, NW, MODE>, dim3((unsigned)grid), dim3(NW * 64), a, g);
  // the dK/dV partials live after the dQ partials
  FwdArgs ak = a;
  ak.part = a.part + (size_t)a.B * a.H * a.g * a.chunks * D;
  if constexpr (kBwdSplitDKV<D>) {
    // dK and dV in two passes (the marks of the dK/dV step bracket both)
    launch(ev ? ev[1].start : nullptr, nullptr, attn_bwd_kernel<D, kBwdDK, NW, MODE>,
           dim3((unsigned)grid), dim3(NW * 64), ak, g);
    launch(nullptr, ev ? ev[1].stop : nullptr, attn_bwd_kernel<D, kBwdDV, NW, MODE>,
           dim3((unsigned)grid), dim3(NW * 64), ak, g);
  } else {
    timed(1, attn_bwd_kernel<D, kBwdDKV, NW, MODE>, dim3((unsigned)grid), dim3(NW * 64), ak, g);
  }
  const long grows = (long)a.B * a.H * a.g;
  if (grows > 0)
    timed(2, bwd_global_combine_kernel<D>, dim3((unsigned)((grows * D + 255) / 256)), dim3(192),
          a, g);
  else if (ev && (hipEventRecord(ev[2].start, s) != hipSuccess ||
                  hipEventRecord(ev[2].stop, s) != hipSuccess))
    return hipErrorUnknown;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_mfma(const FwdArgs& a, const BwdArgs& g, int d, int mode, long grid,
                           hipStream_t s, const LaunchEvents* ev) {
  if (grid <= 0) return hipSuccess;
  if (mode == kBand) {
    if (d == 64) return launch_bwd_d<64, 4, kBand>(a, g, grid, s, ev);
    if (d == 128) return launch_bwd_d<128, 4, kBand>(a, g, grid, s, ev);
  } else if (mode == kLayout && a.block == 64) {
    if (d == 64) return launch_bwd_d<64, 2, kLayout>(a, g, grid, s, ev);
    if (d == 128) return launch_bwd_d<128, 2, kLayout>(a, g, grid, s, ev);
  } else if (mode == kLayout && a.block == 128) {
    if (d == 64) return launch_bwd_d<64, 4, kLayout>(a, g, grid, s, ev);
    if (d == 128) return launch_bwd_d<128, 4, kLayout>(a, g, grid, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace longattn
