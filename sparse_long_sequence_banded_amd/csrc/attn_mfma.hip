// bf16 sparse attention forward on gfx950 matrix cores.
//
// One kernel template serves three workgroup kinds:
//   kBand        a tile of query rows of one (batch, head, dilation residue); walks the key tiles
//                that intersect the window, then the global-key columns.
//   kLayout      one query block of a block-sparse layout; walks the listed key blocks, then the
//                global-key columns.
//   kGlobalRows  the global query rows against one chunk of keys; writes unnormalised partial
//                results that the combine kernel merges.
//
// Attention over a key set is exact masked softmax attention: the window, the global tokens and
// the layout blocks are a set of allowed (query, key) edges, each counted once (Big Bird reading
// notes, sections 3.1 and 3.3).  A dilated window is split into dil independent undilated windows
// over the residue classes i = p (mod dil) (the window skips tokens like a dilated convolution,
// Longformer hub page, section 2), so every key tile here is a plain contiguous or strided band.
// Global-key columns are concatenated after the local keys and share one online softmax with
// them, as the LongT5 guide describes for its side keys (blocking-helpers paragraph).  A global
// key is attended by every query through its column, so window tiles drop global keys (a
// per-tile bit mask shared by the whole workgroup) and layout rows drop global columns that lie
// in one of their blocks; each edge is counted once.
//
// Wave-level math (32x32x16 bf16 MFMA, fp32 accumulate).  A wave owns QB blocks of 32 query rows
// and computes transposed score blocks S^T = K Q^T, so every lane holds the scores of one query
// (its column) for 32 of the 64 keys of a tile; the other 32 sit in lane ^ 32.  Row max and row
// sum are in-lane reductions plus one exchange with lane ^ 32.  The output is kept transposed,
// O^T += V^T P^T, so softmax rescale factors are per lane.
//
// Data movement.  K and V tiles go from memory straight into LDS with 16-byte buffer loads (no
// register staging; the buffer range check turns rows past the sequence end into zeros), two
// stages each, two barriers per tile.  Half of the waves move K, the other half V.  K rows are
// read back as MFMA A operands with 16-byte reads; V stays row-major and its transposed A operand
// is read with the transposing 64-bit LDS read.  Both layouts XOR-swizzle 16-byte chunks by row
// so that the reads of a wave hit distinct banks.

#include <type_traits>

#include <hip/hip_ext.h>

#include "attn_args.h"
#include "mfma_util.h"

namespace longattn {
namespace {

using namespace mfma;

constexpr float kRescaleLog2 = 8.f;  // move the row's reference only when its max exceeds it by > 2^8
constexpr float kFastWeightSum = 65536.f;  // fast path: a lane's 16 weights of a half sum to <= 2^16

// Key tile descriptor, uniform over the workgroup.
struct Tile {
  int gathered;  // 0: row r at position base + kst * r (kst: the workgroup's key stride);
                 // 1: row r is global column base + r
  int base;
  int count;     // rows >= count do not exist (never attended; their loads return zeros or
                 // repeat a valid row)
  int ks0;       // kBand window tiles: residue-subsequence index of row 0
  int lt;        // kBand window tiles: index of the tile within the workgroup's key range
};

// LDS stages of K tiles and of V tiles: two each (loads run one tile ahead) for four-wave
// workgroups; at head dim 64 a workgroup then needs about 36 KB of LDS, so four fit on a CU
// (more resident waves measured faster than a third stage).  Two-wave workgroups (64-row layout
// blocks) take one stage each and are held to 128 VGPRs: about 19 KB of LDS, so eight fit on a
// CU, four waves per SIMD, where two stages would leave two (measured 7% faster on a 64-row
// block layout, a few values spilled).
constexpr int stages_of(int nw) { return nw == 2 ? 1 : 2; }
// Key-padding bits staged in LDS per workgroup: 64-bit words covering 4096 positions.
constexpr int kPadWords = 64;

// LDS of one workgroup (either kind of work uses the same layout).
template <int D, int NS>
struct Smem {
  __attribute__((aligned(1024))) unsigned char stage_k[NS][kKeyTile * D * 2];
  __attribute__((aligned(1024))) unsigned char stage_v[NS][kKeyTile * D * 2];
  int lay_list[256];                            // layout mode: valid key blocks of the row
  __attribute__((aligned(16))) int g_pos[kGlobalCap];  // global columns: positions
  unsigned long long g_valid[kGlobalCap / 64];  // global columns: usable-key bits
  unsigned long long g_bits[kPadWords];         // window mode: global keys among window keys
  unsigned long long pad_bits[kPadWords];       // key padding of the reachable positions
  unsigned long long tmask[kPadWords];          // allowed-key bits of each local tile
  int lay_cnt;
};

// One launch runs the main workgroups (MODE_MAIN) and the global-row partial workgroups
// together.  The main workgroups take the first blockIdx.x values, remapped so that consecutive
// main indices run on one XCD; the global-row workgroups come last in dispatch order, short
// (512-key chunks) and many, so they fill the final round as main workgroups finish instead of
// lengthening it.  The work of one workgroup is a generic lambda over its kind (MODE) and its
// index wg among that kind's workgroups; the kernel arguments stay in the kernel argument
// segment.
template <int D, int NW, int QB, int MODE_MAIN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 2 ? 4 : 1)))
void attn_fwd_kernel(FwdArgs args) {
  __shared__ Smem<D, stages_of(NW)> sm;
  const FwdCore a = args;
  const int total = gridDim.x;
  const int n_rows_wg = a.grid_rows;
  const int n_main_wg = total - n_rows_wg;
  int gi = -1, mi = 0;
  if ((int)blockIdx.x >= n_main_wg) gi = (int)blockIdx.x - n_main_wg;
  else mi = xcd_remap(blockIdx.x, n_main_wg);

  // Main workgroups: batch sample, head, its dilation and the workgroup's index among the head's
  // workgroups, from the per-head workgroup table (read here, in the kernel body, so that the
  // table stays in the kernel argument segment).
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

  // Workgroups flagged by the host raise their waves' priority by the number of tiles left (see
  // balancing_priority): on a 4096-token window launch of one round this takes the kernel from
  // 34.5 to 30.5 us, with the same results bit for bit.
  const bool fair = (int)blockIdx.x >= a.fair_from;
  if (fair) __builtin_amdgcn_s_setprio(3);

  auto body = [&](auto mode_c, const int wg) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int NT = NW * 64;
    constexpr int RW = 32 * QB;        // query rows per wave
    constexpr int QT = NW * RW;        // query rows per workgroup
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int KS = D / 16;         // MFMA k-steps over the head dim
    constexpr int DB = D / 32;         // 32-row blocks of O^T
    constexpr int MAT = kKeyTile * D * 2;
    constexpr int NS = stages_of(NW);
    constexpr int NLOAD = 2 * CH;      // 1 KB direct-load blocks per tile (K blocks, then V)
    constexpr int LPW = NLOAD / NW;    // of which each wave issues
    constexpr int RPB = 64 / CH;       // rows per 1 KB block
    static_assert(NLOAD % NW == 0 && CH % LPW == 0, "each wave loads whole blocks of one matrix");
    static_assert(kGlobalCap % 64 == 0 && NT % 64 == 0, "global staging works in whole waves");
    constexpr bool kHasGlobalCols = MODE != kGlobalRows;

    auto& stage_k = sm.stage_k;
    auto& stage_v = sm.stage_v;
    int* lay_list = sm.lay_list;
    int& lay_cnt = sm.lay_cnt;
    int* g_pos = sm.g_pos;
    unsigned long long* g_valid = sm.g_valid;
    unsigned long long* g_bits = sm.g_bits;
    unsigned long long* pad_bits = sm.pad_bits;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int qj = lane & 31, hh = lane >> 5;

    // ------------------------------------------------------------------ work decomposition
    int b = 0, h = 0, dl = 1, p = 0, np = a.n, q0 = 0, ck = 0, rg = 0;
    if constexpr (MODE == kGlobalRows) {
      const int rgs = (a.g + QT - 1) / QT;
      if (a.rows_by_xcd) {
        // Every (batch, head) takes the same number of main workgroups and the main grid and
        // the (batch, head) count are multiples of 8, so XCD x (blockIdx.x % 8) has run the
        // main work of pairs x*hpx .. x*hpx + hpx - 1, in that order.  Its global-row
        // workgroups (wg % 8 == x) take those pairs' chunks, the most recent pair first and its
        // chunks from the last keys down, which its L2 may still hold (reads below L2 on the
        // 16K dilated workload 169 -> 159 MB, 1-2.5% faster on the three workloads with global
        // tokens).  Any order gives the same results.
        const int per = rgs * a.chunks;    // workgroups per (batch, head)
        const int hpx = (a.B * a.H) >> 3;  // (batch, head) pairs per XCD
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
        q0 = r * QT;
      } else {
        q0 = r * a.block;  // kLayout: query block r (QT == block)
      }
    }
    // key stride of the local tiles (dilation of this head in window mode)
    const int kst = (MODE == kBand) ? min(dl, a.n) : 1;
    const long bh = (long)b * a.H + h;
    const uint16_t* Qb = a.q + bh * a.n * D;
    const uint16_t* Kb = a.k + bh * a.n * D;
    const uint16_t* Vb = a.v + bh * a.n * D;
    const uint8_t* pad = a.kpad ? a.kpad + (long)b * a.n : nullptr;
    const int* gb = a.gidx ? a.gidx + (long)b * a.g : nullptr;

    // ------------------------------------------------------------------ query rows of this lane
    // Lane (qj, hh) holds query row wave*RW + 32qb + qj of the workgroup for every block qb.
    int qpos[QB];  // sequence position, -1 = no such row
    int qsub[QB];  // kBand: residue-subsequence index
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = wave * RW + 32 * qb + qj;
      qpos[qb] = -1;
      qsub[qb] = 0;
      if constexpr (MODE == kBand) {
        qsub[qb] = q0 + qrow;
        if (qsub[qb] < np) qpos[qb] = p + dl * qsub[qb];
      } else if constexpr (MODE == kLayout) {
        qpos[qb] = q0 + qrow;
      } else {
        const int c = rg * QT + qrow;
        if (c < a.g) {
          const int x = gb[c];
          if (x >= 0 && x < a.n) qpos[qb] = x;
        }
      }
    }
    // Q fragments (B operands of the score MFMAs, loaded once) and the global columns' positions.
    // In layout mode both go out before the layout row is compacted, so the three loads' latencies
    // overlap instead of following one another; the other modes load them after the key tiles
    // are known, behind tile 0's loads.
    constexpr int GREG = (kGlobalCap + NT - 1) / NT;
    u32x4 qf[QB][KS];
    int gx[GREG];
    auto load_q = [&]() {
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
        for (int s = 0; s < KS; ++s) {
          qf[qb][s] = u32x4{0, 0, 0, 0};
          if (qpos[qb] >= 0)
            qf[qb][s] = *reinterpret_cast<const u32x4*>(Qb + (long)qpos[qb] * D + 16 * s + 8 * hh);
        }
    };
    auto load_gx = [&]() {
      if constexpr (kHasGlobalCols) {
  #pragma unroll
        for (int i = 0; i < GREG; ++i) {
          const int c = tid + NT * i;
          gx[i] = (a.g > 0 && c < a.g) ? gb[c] : a.n;
        }
      }
    };
    if constexpr (MODE == kLayout) {
      load_gx();
      load_q();
    }

    // ------------------------------------------------------------------ key tiles
    int n_local = 0, k_lo = 0, k_hi = -1;
    constexpr int TPB = QT / kKeyTile;  // layout mode: key tiles per block (QT rows)
    if constexpr (MODE == kBand) {
      if (a.band_on) {
        const int q_last = min(q0 + QT, np) - 1;
        k_lo = max(0, q0 - a.wl);
        k_hi = min(np - 1, q_last + a.wr);
        n_local = (k_hi >= k_lo) ? (k_hi - k_lo + kKeyTile) / kKeyTile : 0;
      }
    } else if constexpr (MODE == kLayout) {
      if (wave == 0) {  // compact the valid block ids of this row into LDS
        const int nb = a.n / a.block;
        const int* row = a.layout + ((long)h * nb + q0 / a.block) * a.max_kb;
        int base = 0;
        for (int e0 = 0; e0 < a.max_kb; e0 += 64) {
          const int e = e0 + lane;
          int id = (e < a.max_kb) ? row[e] : -1;
          if (id >= nb) id = -1;  // out-of-range ids are ignored rather than read
          const unsigned long long m = __ballot(id >= 0);
          if (id >= 0) lay_list[base + __popcll(m & ((1ull << lane) - 1ull))] = id;
          base += __popcll(m);
        }
        if (lane == 0) lay_cnt = base;
      }
      __syncthreads();
      n_local = lay_cnt * TPB;
    } else {
      const int c0 = ck * a.chunk_keys;
      const int c1 = min(a.n, c0 + a.chunk_keys);
      n_local = (c1 > c0) ? (c1 - c0 + kKeyTile - 1) / kKeyTile : 0;
      k_lo = c0;
      k_hi = c1 - 1;
    }
    const int n_gtiles = (kHasGlobalCols && a.g > 0) ? (a.g + kKeyTile - 1) / kKeyTile : 0;
    const int n_tiles = n_local + n_gtiles;
    // At head dim 64, window mode walks its key tiles in a rotated order: step t takes the tile
    // whose index in the residue subsequence, (k_lo / 64) + lt, is congruent to t modulo
    // n_local.  Neighbouring query tiles (whose key ranges overlap in all but two tiles) then
    // read the same K/V tile at the same step instead of two steps apart, so the re-reads hit
    // the XCD's L2 (about a quarter less read traffic below L2 on a 16K-token window of 256 keys
    // each side, and about 1% faster).  The softmax does not depend on the order of the keys.
    // The head-dim-128 kernel keeps the natural order: there the added index arithmetic alone
    // (measured with the order unchanged, same output bits) made the 32K causal window 1.5%
    // slower.
    int rot = 0;
    if constexpr (MODE == kBand && D == 64) {
      if (n_local > 0) rot = (n_local - (k_lo / kKeyTile) % n_local) % n_local;
    }

    auto tile_of = [&](int t) -> Tile {
      Tile T;
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
        T.ks0 = k_lo + T.lt * kKeyTile;
        T.base = p + dl * T.ks0;
        T.count = min(kKeyTile, np - T.ks0);
      } else if constexpr (MODE == kLayout) {
        T.gathered = 0;
        T.lt = t;
        T.base = lay_list[t / TPB] * a.block + (t % TPB) * kKeyTile;
        T.count = kKeyTile;
      } else {
        T.gathered = 0;
        T.lt = t;
        T.base = k_lo + t * kKeyTile;
        T.count = min(kKeyTile, k_hi + 1 - T.base);
      }
      return T;
    };

    // ------------------------------------------------------------------ tile loading
    // Wave w moves the 1 KB blocks w*LPW .. w*LPW + LPW - 1 of a tile: all of one matrix (K for
    // the first half of the waves, the "K waves", V for the rest).  Block `sub` of a matrix holds
    // rows RPB*sub .. RPB*sub + RPB - 1; lane l moves row RPB*sub + l/CH, 16-byte chunk l%CH, to
    // LDS byte sub*1024 + 16*l (the chunk's swizzled slot in that row).
    const int mat = (wave * LPW) / CH;
    const int sub0 = (wave * LPW) % CH;
    auto ld_row = [&](int j) -> int { return (sub0 + j) * RPB + lane / CH; };
    auto ld_col = [&](int j) -> int {
      const int row = ld_row(j);
      return 8 * ((lane % CH) ^ (mat == 0 ? swz_k<D>(row) : swz_v<D>(row)));
    };
    // byte offsets of this lane's chunks within a local tile starting at row 0 (rows past the
    // sequence end land at or beyond the resource size, so they read zeros)
    uint32_t voff[LPW];
  #pragma unroll
    for (int j = 0; j < LPW; ++j)
      voff[j] = (uint32_t)(min((long)ld_row(j) * kst, (long)a.n) * D + ld_col(j)) * 2u;
    const uint16_t* msrc = (mat == 0) ? Kb : Vb;
    auto issue = [&](unsigned char* st, const Tile& T) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(st + sub0 * 1024));
      if (kHasGlobalCols && T.gathered) {
        const u32x4 rs = buf_rsrc(msrc, (uint32_t)a.n * D * 2u);
  #pragma unroll
        for (int j = 0; j < LPW; ++j) {
          const int pos = g_pos[T.base + min(ld_row(j), T.count - 1)];
          lds_dma16(rs, (uint32_t)(pos * D + ld_col(j)) * 2u, dst + 1024 * j);
        }
      } else {
        const u32x4 rs = buf_rsrc(msrc + (long)T.base * D, (uint32_t)(a.n - T.base) * D * 2u);
  #pragma unroll
        for (int j = 0; j < LPW; ++j) lds_dma16(rs, voff[j], dst + 1024 * j);
      }
    };
    const bool kwave = mat == 0;
    // Global column positions are loaded first (the staging below needs them and, with key
    // padding, loads a pad byte at each), then tile 0's loads go out when it is a local tile (it
    // needs nothing from the staging), so their latency overlaps that of the Q fragments and the
    // staging.
    if constexpr (MODE != kLayout) load_gx();
    if (n_local > 0) issue(kwave ? stage_k[0] : stage_v[0], tile_of(0));

    if constexpr (MODE != kLayout) load_q();
    const float c2 = a.scale_log2;

    // ------------------------------------------------------------------ staging in LDS
    // Global-key columns: position and validity, once per workgroup.  A usable global key is
    // attended through the global-column tiles by every query, so in window mode the local tiles
    // drop it (each edge is counted once): g_bits marks the global keys among the window keys,
    // bit i of word t for residue index k_lo + 64t + i, when the window range fits; otherwise
    // each local tile searches the sorted positions.
    const bool gbits_staged = MODE == kBand && n_gtiles > 0 && n_local <= kPadWords;
    if constexpr (kHasGlobalCols) {
      if (n_gtiles > 0) {
        if constexpr (MODE == kBand) {
          if (gbits_staged) {
            for (int w = tid; w < n_local; w += NT) g_bits[w] = 0ull;
            __syncthreads();
          }
        }
  #pragma unroll
        for (int i = 0; i < GREG; ++i) {
          const int c = tid + NT * i;
          if (NT * (i + 1) > kGlobalCap && c >= kGlobalCap) continue;  // whole waves past the cap
          const int x = gx[i];
          bool ok = x >= 0 && x < a.n;         // a usable key: in range and not padded
          if (ok && pad) ok = pad[x] == 0;
          const int pos = min(max(x, 0), a.n);  // keeps the positions ascending
          if constexpr (MODE == kLayout) {
            // a global key inside one of this row's layout blocks is attended through the block
            const int blk = pos / a.block;
            for (int e = 0; e < lay_cnt; ++e) ok = ok && (lay_list[e] != blk);
          }
          if constexpr (MODE == kBand) {
            const int rel = pos - p;
            if (gbits_staged && ok && rel >= 0 && rel % dl == 0) {
              const int j = rel / dl - k_lo;
              if (j >= 0 && j < kKeyTile * n_local) atomicOr(&g_bits[j >> 6], 1ull << (j & 63));
            }
          }
          g_pos[c] = pos;
          const unsigned long long vm = __ballot(ok);
          if (lane == 0) g_valid[c >> 6] = vm;
        }
      }
    }
    // Key padding of the positions the local tiles can reach, as bits (bit i of word w: position
    // pad_lo + 64w + i is a usable key), when they fit; otherwise each tile reads its pad bytes.
    int pad_lo = 0;
    bool pad_staged = false;
    if (pad && n_local > 0) {
      long lo, hi;
      if constexpr (MODE == kBand) {
        lo = p + (long)dl * k_lo;
        hi = min((long)a.n - 1, p + (long)dl * (k_lo + (long)kKeyTile * n_local - 1));
      } else if constexpr (MODE == kLayout) {
        lo = 0;
        hi = a.n - 1;
      } else {
        lo = k_lo;
        hi = k_hi;
      }
      lo &= ~63L;
      const long words = ((hi - lo) >> 6) + 1;
      pad_staged = words <= kPadWords;
      pad_lo = (int)lo;
      if (pad_staged) {
        // four words per wave per round, their loads issued together
        for (int w0 = wave; w0 < (int)words; w0 += 4 * NW) {
          int pb[4];
  #pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int pos = pad_lo + 64 * (w0 + NW * u) + lane;
            pb[u] = (w0 + NW * u < (int)words && pos < a.n) ? pad[pos] : 1;
          }
  #pragma unroll
          for (int u = 0; u < 4; ++u) {
            const unsigned long long m = __ballot(pb[u] == 0);
            if (lane == 0 && w0 + NW * u < (int)words) pad_bits[w0 + NW * u] = m;
          }
        }
      }
    }
    // Consume the fragments here so that the compiler waits for these loads before the tile loop;
    // otherwise it waits for them (vmcnt(0), which also drains the K/V prefetch) inside the loop.
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
      for (int s = 0; s < KS; ++s) asm volatile("" : : "v"(qf[qb][s]));
    __syncthreads();
    // a gathered first tile (its rows come from the staged positions)
    if (n_local == 0 && n_tiles > 0) issue(kwave ? stage_k[0] : stage_v[0], tile_of(0));


    // window mode: bits of the usable global keys among the rows of local tile t
    auto global_keys = [&](const Tile& T, int t) -> unsigned long long {
      if (n_gtiles == 0) return 0ull;
      if (gbits_staged) return g_bits[t];
      const bool in = lane < T.count;
      const int pos = in ? T.base + kst * lane : 0;
      int c = -1;  // last column with position <= pos (positions ascend)
  #pragma unroll
      for (int step = kGlobalCap; step > 0; step >>= 1)
        if (c + step < a.g && g_pos[c + step] <= pos) c += step;
      const bool hit = in && c >= 0 && g_pos[c] == pos && ((g_valid[c >> 6] >> (c & 63)) & 1ull);
      return __ballot(hit);
    };
    // allowed-key bits of a local tile (bit r: row r exists and is not padded)
    auto local_valid = [&](const Tile& T) -> unsigned long long {
      if (!pad) return T.count >= 64 ? ~0ull : ((1ull << T.count) - 1ull);
      const bool in = lane < T.count;
      const long pos = in ? (long)T.base + (long)kst * lane : 0;
      bool ok;
      if (pad_staged) {
        const int rel = in ? (int)(pos - pad_lo) : 0;
        ok = in && ((pad_bits[rel >> 6] >> (rel & 63)) & 1ull);
      } else {
        ok = in && pad[pos] == 0;
      }
      return __ballot(ok);
    };
    // The allowed-key bits of every local tile (existing, not padded, and in window mode not a
    // global key), computed once per workgroup (tile lt by wave lt % NW) when they fit and take
    // more than the tile's count and one staged word; the first tile barrier of the loop
    // publishes them.
    const bool tmask_staged =
        n_local <= kPadWords && (pad != nullptr || (n_gtiles > 0 && !gbits_staged && MODE == kBand));
    if (tmask_staged) {
      for (int t = wave; t < n_local; t += NW) {
        int lt = t;
        if constexpr (MODE == kBand && D == 64) lt = t + rot < n_local ? t + rot : t + rot - n_local;
        const Tile T = tile_of(t);
        unsigned long long m = local_valid(T);
        if constexpr (MODE == kBand) m &= ~global_keys(T, lt);
        if (lane == 0) sm.tmask[lt] = m;
      }
    }

    // ------------------------------------------------------------------ per-lane LDS read offsets
    // K operand of S^T for key block kb, k-step ks: row 32kb + qj, logical chunk 2ks + hh.
    // V^T operand for 16-key group t, d block db, half r: transposing read; lane l of 16-lane group
    // G = l/16 supplies row 16t + 8r + 4(l/32) + (l%16)/4 at d = 32db + 16(G%2) + 4(l%4) and gets
    // V[16t + 8r + 4(l/32) + e][32db + l%32], e = 0..3.
    const int ksw = swz_k<D>(qj);  // the same for rows qj and 32 + qj
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

    // ------------------------------------------------------------------ running state
    // Per row: ref = the exponent offset all weights of the row are taken against (log2 units),
    // has = some allowed key has been seen, o = the sum of value rows weighted by the bf16-rounded
    // weights 2^(c2 s - ref) (transposed: o[qb][db][r] is column 32db + 8(r/4) + 4hh + r%4),
    // l = the sum of those rounded weights: o / l is the output, so the weights that multiply the
    // value rows add up to one and a row dominated by a few keys carries no rounding bias.
    f32x16 o[QB][DB];
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
      for (int db = 0; db < DB; ++db)
  #pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    float ref[QB], l_run[QB];
    bool has[QB];
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ref[qb] = 0.f;
      l_run[qb] = 0.f;
      has[qb] = false;
    }

    // wave row range (kBand tile skipping)
    const int w_first = q0 + wave * RW;
    const int w_last = (MODE == kBand) ? min(w_first + RW - 1, np - 1) : w_first + RW - 1;
    bool wave_rows;
    if constexpr (MODE == kBand) wave_rows = w_first < np;
    else if constexpr (MODE == kLayout) wave_rows = true;
    else wave_rows = (rg * QT + wave * RW) < a.g;

    // ------------------------------------------------------------------ one tile
    // ---- raw scores S^T = K Q^T of both 32-key halves of a K tile, for every query block
    auto scores = [&](const unsigned char* st, f32x16 (&sc)[2][QB]) {
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][qb][r] = 0.f;
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(st + koff[ks] + kb * 32 * (2 * D));
  #pragma unroll
          for (int qb = 0; qb < QB; ++qb) sc[kb][qb] = mfma_32x32x16(kf, qf[qb][ks], sc[kb][qb]);
        }
        // the first half's chain goes out whole before the second's, so its softmax can start
        // while the matrix cores work on the second half (interleaved chains finish together)
        if (kb == 0) __builtin_amdgcn_sched_barrier(0);
      }
    };
    // ---- masks, online softmax step and O^T += V^T P^T for one tile whose scores are in sc.
    // Per-element masks (key validity bits and, in window mode, the band edges) are applied only
    // when some key of the tile is excluded for some row of the wave; interior tiles skip them.
    auto finish = [&](f32x16 (&sc)[2][QB], const unsigned char* st, const Tile& T,
                      unsigned long long vmask, bool need_band) {
      // ---- masks.  Register r of half kb holds key 32kb + 8(r/4) + 4hh + r%4, i.e. bit
      // 8(r/4) + r%4 of w = (the tile's allowed keys for this lane's query) >> (32kb + 4hh).
      if (need_band || vmask != ~0ull) {
        const float ninf = neg_inf();
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          unsigned long long m = vmask >> (4 * hh);
          if (need_band) {
            // keys k with qs - wl <= ks0 + k <= qs + wr, shifted by this lane's 4*hh
            const int lo = qsub[qb] - a.wl - T.ks0 - 4 * hh;
            const int hi = qsub[qb] + a.wr - T.ks0 - 4 * hh;
            unsigned long long bm = 0ull;
            if (hi >= 0 && lo <= 63) {
              const int lc = max(lo, 0), hc = min(hi, 63);
              bm = (~0ull >> (63 - (hc - lc))) << lc;
            }
            m &= bm;
          }
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            uint32_t w = (uint32_t)(m >> (32 * kb));
            asm("" : "+v"(w));  // per-lane word: the selects below stay two VALU ops each
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              sc[kb][qb][r] = keep_if_bit(sc[kb][qb][r], w, 8 * (r >> 2) + (r & 3), ninf);
          }
        }
      }

      // ---- online softmax step, one 32-key half at a time.  Weights are 2^(c2 s - ref), c2 =
      // scale * log2(e), against a per-row reference ref; the final normalisation by l makes the
      // result exact for any reference that keeps the weights finite and not all underflowing.
      // Fast path (rows that already have a reference): exponentiate against it without a row
      // max and accept when every lane's 16 weights sum to at most 2^16 (so no weight exceeds
      // 2^16 and nothing overflows).  Otherwise (a row's first allowed key, or a score far above
      // the reference) take the half's row max: a row moves its reference to that max when it
      // has none yet or when the max exceeds ref by more than 2^8, and the weights are redone.
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t pk[QB][8];
        float part[QB];
        auto exponentiate = [&]() {
  #pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float nr = -ref[qb];
            float la = 0.f, lb = 0.f;
  #pragma unroll
            for (int r = 0; r < 16; r += 4) {
              const float p0 = exp2_fast(__builtin_fmaf(sc[kb][qb][r], c2, nr));
              const float p1 = exp2_fast(__builtin_fmaf(sc[kb][qb][r + 1], c2, nr));
              const float p2 = exp2_fast(__builtin_fmaf(sc[kb][qb][r + 2], c2, nr));
              const float p3 = exp2_fast(__builtin_fmaf(sc[kb][qb][r + 3], c2, nr));
              pk[qb][r >> 1] = pack_bf16x2(p0, p1);
              pk[qb][(r >> 1) + 1] = pack_bf16x2(p2, p3);
              la = add_bf16x2(pk[qb][r >> 1], la);  // the rounded weights the PV products use
              lb = add_bf16x2(pk[qb][(r >> 1) + 1], lb);
            }
            part[qb] = la + lb;
          }
        };
        bool no_ref = false;
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) no_ref = no_ref | !has[qb];
        bool slow = __builtin_amdgcn_ballot_w64(no_ref) != 0ull;
        if (!slow) {
          exponentiate();
          bool over = false;
  #pragma unroll
          for (int qb = 0; qb < QB; ++qb) over = over | !(part[qb] <= kFastWeightSum);
          slow = __builtin_amdgcn_ballot_w64(over) != 0ull;
        }
        if (slow) {
          float xm[QB];
          bool need[QB];
          bool need_any = false;
  #pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const f32x16& u = sc[kb][qb];
            float x0 = __builtin_fmaxf(__builtin_fmaxf(u[0], u[1]), u[2]);
            float x1 = __builtin_fmaxf(__builtin_fmaxf(u[3], u[4]), u[5]);
            x0 = __builtin_fmaxf(__builtin_fmaxf(x0, u[6]), u[7]);
            x1 = __builtin_fmaxf(__builtin_fmaxf(x1, u[8]), u[9]);
            x0 = __builtin_fmaxf(__builtin_fmaxf(x0, u[10]), u[11]);
            x1 = __builtin_fmaxf(__builtin_fmaxf(x1, u[12]), u[13]);
            x0 = __builtin_fmaxf(__builtin_fmaxf(x0, u[14]), __builtin_fmaxf(x1, u[15]));
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0),
                                                             __float_as_uint(x0), false, false);
            const float x = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c2;
            xm[qb] = x;
            need[qb] = (x != neg_inf()) & (!has[qb] | (x - ref[qb] > kRescaleLog2));
            need_any = need_any | need[qb];
          }
          if (__builtin_amdgcn_ballot_w64(need_any) != 0ull) {
            // per lane, the new reference is the row max if the row moves, else the old one
  #pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const float nref = need[qb] ? xm[qb] : ref[qb];
              const float alpha = has[qb] ? exp2_fast(ref[qb] - nref) : 1.f;  // old weights
              ref[qb] = nref;
              has[qb] = has[qb] || need[qb];
              l_run[qb] *= alpha;
  #pragma unroll
              for (int db = 0; db < DB; ++db)
  #pragma unroll
                for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
            }
          }
          exponentiate();
        }
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] += part[qb];
        // ---- O^T += V^T P^T for the 16-key groups 2kb, 2kb+1
  #pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
          const int g = 2 * kb + gh;
  #pragma unroll
          for (int db = 0; db < DB; ++db) {
            const unsigned char* vp = st + voffs[db] + 16 * g * (2 * D);
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp));
            const s16x4 v1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp + 8 * (2 * D)));
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
  #pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const u32x4 bp = {pk[qb][4 * gh + 0], pk[qb][4 * gh + 1], pk[qb][4 * gh + 2],
                                pk[qb][4 * gh + 3]};
              o[qb][db] = mfma_32x32x16(va, bp, o[qb][db]);
            }
          }
        }
      }
    };
    // Does tile T hold keys in reach of this wave's rows (window mode), and do band edges cut it?
    auto reach = [&](const Tile& T, bool& need_band) -> bool {
      need_band = false;
      if (!wave_rows) return false;
      if constexpr (MODE == kBand) {
        if (!T.gathered) {
          const int kf = T.ks0, kl = T.ks0 + kKeyTile - 1;
          if (kl < w_first - a.wl || kf > w_last + a.wr) return false;
          need_band = !(kf >= w_last - a.wl && kl <= w_first + a.wr);
        }
      }
      return true;
    };

    // ------------------------------------------------------------------ tile loop
    // Two stages: tile t lives in stage t % 2.  Step t: a barrier retires every read of tile
    // t-1, whose stage then takes tile t+1's loads; each wave then waits for its own loads of
    // tile t only (tile t+1's stay in flight: loads complete in issue order), and a second
    // barrier makes tile t visible to every wave.  Issuing tile t+1 before waiting for tile t
    // keeps two tiles in flight whenever a load is late.  One stage: the barrier that retires
    // tile t-1 precedes tile t's loads, which are waited for at once (other workgroups on the CU
    // cover the wait).  Tile 0 was issued above.
    if (n_tiles > 0) {
      int st = 0;  // stage of tile t
      for (int t = 0; t < n_tiles; ++t) {
        if (fair) balancing_priority(n_tiles - t);
        if constexpr (NS == 1) {
          if (t > 0) {
            __syncthreads();  // every wave is done with tile t-1: the stage may be refilled
            issue(kwave ? stage_k[0] : stage_v[0], tile_of(t));
          }
          wait_vmcnt<0>();
        } else {
          if (t > 0) __syncthreads();  // every wave is done with tile t-1: its stage may be refilled
          if (t + 1 < n_tiles) issue(kwave ? stage_k[st ^ 1] : stage_v[st ^ 1], tile_of(t + 1));
          if (t + 1 < n_tiles) wait_vmcnt<LPW>();  // tile t landed; tile t+1 stays in flight
          else wait_vmcnt<0>();
        }
        __syncthreads();  // tile t visible to every wave
        const Tile T = tile_of(t);
        bool need_band = false;
        if (reach(T, need_band)) {
          unsigned long long vmask;
          if (T.gathered) vmask = g_valid[T.base >> 6];
          else if (tmask_staged) vmask = sm.tmask[T.lt];
          else if constexpr (MODE == kBand) vmask = local_valid(T) & ~global_keys(T, T.lt);
          else vmask = local_valid(T);
          f32x16 sc[2][QB];
          scores(stage_k[st], sc);
          finish(sc, stage_v[st], T, vmask, need_band);
        }
        if constexpr (NS == 2) st ^= 1;
      }
    }

    // ------------------------------------------------------------------ epilogue
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = l_run[qb] + __uint_as_float(__shfl_xor(__float_as_uint(l_run[qb]), 32));
      if (qpos[qb] < 0) continue;
      if constexpr (MODE == kGlobalRows) {
        const int c = rg * QT + wave * RW + 32 * qb + qj;
        const long slot = (bh * a.g + c) * a.chunks + ck;
        float* po = a.part + slot * D;
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d = 32 * db + 8 * rq + 4 * hh;
            *reinterpret_cast<float4*>(po + d) =
                make_float4(o[qb][db][4 * rq], o[qb][db][4 * rq + 1], o[qb][db][4 * rq + 2],
                            o[qb][db][4 * rq + 3]);
          }
        if (hh == 0) {
          float* pml = a.part + (long)a.B * a.H * a.g * a.chunks * D + slot * 2;
          pml[0] = has[qb] ? ref[qb] : neg_inf();
          pml[1] = l_tot;
        }
      } else {
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        uint16_t* orow = a.out + (bh * a.n + qpos[qb]) * D;
        // elementwise output gate (gated attention): out *= sigmoid(gate logits)
        const uint16_t* grow = a.gate ? a.gate + (bh * a.n + qpos[qb]) * D : nullptr;
  #pragma unroll
        for (int db = 0; db < DB; ++db)
  #pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d = 32 * db + 8 * rq + 4 * hh;
            float y0 = o[qb][db][4 * rq] * inv, y1 = o[qb][db][4 * rq + 1] * inv;
            float y2 = o[qb][db][4 * rq + 2] * inv, y3 = o[qb][db][4 * rq + 3] * inv;
            if (grow) {
              const u32x2 gw = *reinterpret_cast<const u32x2*>(grow + d);
              y0 *= sigmoid_fast(bf16_lo(gw[0]));
              y1 *= sigmoid_fast(bf16_hi(gw[0]));
              y2 *= sigmoid_fast(bf16_lo(gw[1]));
              y3 *= sigmoid_fast(bf16_hi(gw[1]));
            }
            u32x2 w;
            w[0] = pack_bf16x2(y0, y1);
            w[1] = pack_bf16x2(y2, y3);
            *reinterpret_cast<u32x2*>(orow + d) = w;
          }
        if (a.lse && hh == 0)
          a.lse[bh * a.n + qpos[qb]] =
              (l_tot > 0.f) ? (ref[qb] + __log2f(l_tot)) * kLn2 : neg_inf();
      }
    }
  };
  if (gi >= 0) body(std::integral_constant<int, kGlobalRows>{}, gi);
  else body(std::integral_constant<int, MODE_MAIN>{}, mi);
}

// Merge the per-chunk partials of every global row and write its output and lse.
// One 256-thread workgroup per (batch, head, global row).  Thread t owns output columns
// 4(t % (D/4)) .. +3 of the chunks t / (D/4), + 256/(D/4), ...: every partial load of the row is
// in flight at once.  Each thread merges its chunks against its own running maximum; the chunk
// groups are then merged through LDS (one load round, one LDS round).
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void global_combine_kernel(FwdArgs args) {
  constexpr int QPR = D / 4;                    // column quads per row
  constexpr int CG = kCombineThreads / QPR;     // chunk groups
  constexpr float kNegInf = -__builtin_inff();
  __shared__ float4 part[CG][QPR];
  __shared__ float gmax[CG], gsum[CG];
  const FwdCore a = args;
  const int t = threadIdx.x;
  const long rows = (long)a.B * a.H * a.g;
  const long row = blockIdx.x;
  const long bh = row / a.g;
  const int c = (int)(row - bh * a.g);
  const int b = (int)(bh / a.H);
  const int pos = a.gidx[(long)b * a.g + c];
  if (pos < 0 || pos >= a.n) return;  // out-of-range global index: nothing to write (uniform)
  const int K = a.chunks;
  const float* po = a.part + row * K * D;
  const float* pml = a.part + rows * K * D + row * K * 2;
  const int cg = t / QPR, cq = t % QPR;
  float m = kNegInf, l = 0.f;                 // running max and normaliser of this thread
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // This thread's chunks k = cg, cg + CG, ... in batches of KB whose loads all go out before any
  // is used (an index past the last chunk reads the last one and is then skipped), merged in
  // chunk order.
  constexpr int KB = 4;
  for (int k0 = cg; k0 < K; k0 += KB * CG) {
    float mk[KB], lk[KB];
    float4 v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = min(k0 + u * CG, K - 1);
      mk[u] = pml[2 * k];
      lk[u] = pml[2 * k + 1];
      v[u] = *reinterpret_cast<const float4*>(po + (long)k * D + 4 * cq);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      // past the last chunk, or a chunk with no key (o = 0, l = 0)
      if (k0 + u * CG >= K || mk[u] == kNegInf) continue;
      const float mn = fmaxf(m, mk[u]);
      const float s_old = (m == kNegInf) ? 0.f : exp2f(m - mn), s_new = exp2f(mk[u] - mn);
      acc.x = acc.x * s_old + v[u].x * s_new;
      acc.y = acc.y * s_old + v[u].y * s_new;
      acc.z = acc.z * s_old + v[u].z * s_new;
      acc.w = acc.w * s_old + v[u].w * s_new;
      l = l * s_old + lk[u] * s_new;
      m = mn;
    }
  }
  part[cg][cq] = acc;
  if (cq == 0) {
    gmax[cg] = m;
    gsum[cg] = l;
  }
  __syncthreads();
  if (t < QPR) {
    float M = kNegInf;
    for (int gi = 0; gi < CG; ++gi) M = fmaxf(M, gmax[gi]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != kNegInf) {
      for (int gi = 0; gi < CG; ++gi) {
        if (gmax[gi] == kNegInf) continue;
        const float w = exp2f(gmax[gi] - M);
        const float4 v = part[gi][t];
        o.x += w * v.x;
        o.y += w * v.y;
        o.z += w * v.z;
        o.w += w * v.w;
        L += w * gsum[gi];
      }
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    uint16_t* orow = a.out + (bh * a.n + pos) * D + 4 * t;
    float y[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
    if (a.gate) {  // elementwise output gate
      const u32x2 gw = *reinterpret_cast<const u32x2*>(a.gate + (bh * a.n + pos) * D + 4 * t);
      y[0] *= sigmoid_fast(bf16_lo(gw[0]));
      y[1] *= sigmoid_fast(bf16_hi(gw[0]));
      y[2] *= sigmoid_fast(bf16_lo(gw[1]));
      y[3] *= sigmoid_fast(bf16_hi(gw[1]));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = __builtin_bit_cast(uint16_t, (__bf16)y[e]);
    if (a.lse && t == 0) a.lse[bh * a.n + pos] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
  }
}

// The same merge when a row has at most kFlatChunks chunks: one thread per (global row, column
// quad) merges all of the row's chunks itself (the chunks' maximum first, then the weighted sums
// in chunk order), every load in one batch and no LDS round, 256-thread workgroups over all rows.
// The partials are loaded before the row's global index is checked (they exist whatever it is),
// so the two loads overlap.
// On a 4K-token block layout with 128 global tokens (3072 rows of 8 chunks) this takes the merge
// from 5.5 to 4.1 us; the per-row form stays for longer rows, whose chunks it spreads over
// threads.
constexpr int kFlatChunks = 8;
template <int D>
__global__ __launch_bounds__(256) void global_combine_flat_kernel(FwdArgs args) {
  constexpr int QPR = D / 4;
  const FwdCore a = args;
  const long rows = (long)a.B * a.H * a.g;
  const long it = (long)blockIdx.x * 256 + threadIdx.x;
  if (it >= rows * QPR) return;
  const long row = it / QPR;
  const int cq = (int)(it - row * QPR);
  const long bh = row / a.g;
  const int c = (int)(row - bh * a.g);
  const int b = (int)(bh / a.H);
  const int pos = a.gidx[(long)b * a.g + c];
  const int K = a.chunks;
  const float* po = a.part + row * K * D + 4 * cq;
  const float* pml = a.part + rows * K * D + row * K * 2;
  float2 ml[kFlatChunks];
  float4 v[kFlatChunks];
#pragma unroll
  for (int k = 0; k < kFlatChunks; ++k) {
    const int kk = min(k, K - 1);
    ml[k] = *reinterpret_cast<const float2*>(pml + 2 * kk);
    v[k] = *reinterpret_cast<const float4*>(po + (long)kk * D);
  }
  float m = neg_inf();
#pragma unroll
  for (int k = 0; k < kFlatChunks; ++k)
    if (k < K) m = fmaxf(m, ml[k].x);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.f;
  if (m != neg_inf()) {
#pragma unroll
    for (int k = 0; k < kFlatChunks; ++k) {
      if (k >= K || ml[k].x == neg_inf()) continue;
      const float w = exp2f(ml[k].x - m);
      acc.x += w * v[k].x;
      acc.y += w * v[k].y;
      acc.z += w * v[k].z;
      acc.w += w * v[k].w;
      l += w * ml[k].y;
    }
  }
  if (pos < 0 || pos >= a.n) return;  // an out-of-range global index: nothing to write
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  float y[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  const long off = (bh * a.n + pos) * D + 4 * cq;
  if (a.gate) {
    const u32x2 gw = *reinterpret_cast<const u32x2*>(a.gate + off);
    y[0] *= sigmoid_fast(bf16_lo(gw[0]));
    y[1] *= sigmoid_fast(bf16_hi(gw[0]));
    y[2] *= sigmoid_fast(bf16_lo(gw[1]));
    y[3] *= sigmoid_fast(bf16_hi(gw[1]));
  }
  u32x2 w;
  w[0] = pack_bf16x2(y[0], y[1]);
  w[1] = pack_bf16x2(y[2], y[3]);
  *reinterpret_cast<u32x2*>(a.out + off) = w;
  if (a.lse && cq == 0) a.lse[bh * a.n + pos] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : neg_inf();
}

template <int D, int NW, int QB, int MODE>
hipError_t launch_one(const FwdArgs& a0, long grid, hipStream_t s, const LaunchEvents& ev) {
  if (grid <= 0) return hipSuccess;
  static std::atomic<long> cap_cache[kMaxDevices];
  const long cap = resident_capacity(reinterpret_cast<const void*>(&attn_fwd_kernel<D, NW, QB, MODE>),
                                     NW * 64, s, cap_cache);
  FwdArgs a = a0;
  a.fair_from = balancing_from(grid, cap);
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, MODE>), dim3((unsigned)grid),
                          dim3(NW * 64), 0, s, ev.start, ev.stop, 0, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, MODE>), dim3((unsigned)grid), dim3(NW * 64),
                       0, s, a);
  return hipGetLastError();
}

}  // namespace

// Query rows per workgroup of the main work: 128 in window mode (four waves of one 32-row
// block), the block size in layout mode.  The global-row workgroups of the same launch take as
// many global rows (one 32-row block per wave).
int main_rows_per_workgroup(int mode, int d, int block) {
  (void)d;
  return mode == kLayout ? block : 128;
}

hipError_t launch_attention(const FwdArgs& a, int d, int mode, long grid, hipStream_t s,
                            const LaunchEvents& ev) {
  if (mode == kBand) {
    if (d == 64) return launch_one<64, 4, 1, kBand>(a, grid, s, ev);
    if (d == 128) return launch_one<128, 4, 1, kBand>(a, grid, s, ev);
  } else if (mode == kLayout) {
    if (a.block == 64) {
      if (d == 64) return launch_one<64, 2, 1, kLayout>(a, grid, s, ev);
      if (d == 128) return launch_one<128, 2, 1, kLayout>(a, grid, s, ev);
    } else if (a.block == 128) {
      if (d == 64) return launch_one<64, 4, 1, kLayout>(a, grid, s, ev);
      if (d == 128) return launch_one<128, 4, 1, kLayout>(a, grid, s, ev);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_global_combine(const FwdArgs& a, int d, hipStream_t s, const LaunchEvents& ev) {
  const long rows = (long)a.B * a.H * a.g;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(kCombineThreads);
  auto launch = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, a);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
  };
  if (a.chunks <= kFlatChunks) {
    const dim3 fgrid((unsigned)((rows * (d / 4) + 255) / 256)), fblock(256);
    auto launchf = [&](auto kernel) {
      if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kernel, fgrid, fblock, 0, s, ev.start, ev.stop, 0, a);
      else
        hipLaunchKernelGGL(kernel, fgrid, fblock, 0, s, a);
    };
    if (d == 64) launchf(global_combine_flat_kernel<64>);
    else if (d == 128) launchf(global_combine_flat_kernel<128>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (d == 64) launch(global_combine_kernel<64>);
  else if (d == 128) launch(global_combine_kernel<128>);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace longattn
