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
// them, as the LongT5 guide describes for its side keys (blocking-helpers paragraph).
//
// Wave-level math (32x32x16 bf16 MFMA, fp32 accumulate).  A wave owns QB blocks of 32 query rows
// and computes transposed score blocks S^T = K Q^T, so every lane holds the scores of one query
// (its column) for 32 of the 64 keys of a tile; the other 32 sit in lane ^ 32.  Row max and row
// sum are in-lane reductions plus one exchange with lane ^ 32.  The output is kept transposed,
// O^T += V^T P^T, so softmax rescale factors are per lane.
//
// Data movement.  K and V tiles go from memory straight into LDS with 16-byte direct loads (no
// register staging), double-buffered, one barrier per tile.  K rows are read back as MFMA A
// operands with 16-byte reads; V stays row-major and its transposed A operand is read with the
// transposing 64-bit LDS read.  Both layouts XOR-swizzle 16-byte chunks by row so that the reads
// of a wave hit distinct banks.

#include <type_traits>

#include "attn_args.h"

namespace longattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kJrNone = -(1 << 29);  // "this global key is not in the query's residue class"
constexpr float kRescaleLog2 = 8.f;  // rescale only when the running max grows by > 2^8

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0; the other counters are left
// at their maxima), then barrier.  The explicit wait is required: the workgroup fence inside
// __syncthreads() only orders this wave's LDS stores and does not count the LDS writes of
// direct loads, so the compiler may otherwise reach the barrier with those loads in flight.
__device__ __forceinline__ void wait_loads_then_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt(0) expcnt(7) lgkmcnt(15)
  __syncthreads();
}

// Logical workgroup id such that consecutive ids run on the same XCD.  Workgroups are handed to
// the 8 XCDs round robin, so neighbouring query tiles (which re-read the same K/V rows) would
// otherwise land in 8 different L2 caches.  This is a bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int x, int G) {
  const int q = G >> 3, r = G & 7;
  const int xcd = x & 7, idx = x >> 3;
  return xcd * q + min(xcd, r) + idx;
}

// 16-byte chunk swizzles.  K: 16 consecutive rows reading the same logical chunk land in 16
// distinct bank groups (64 banks of 4 bytes).  V: the transposing read of 4 consecutive rows x
// 64 bytes by 32 lanes lands in distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 64) return (row >> 1) & 7;
  else return row & 15;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 64) return ((row >> 1) & 1) << 2;
  else return (row & 3) << 2;
}

// Key tile descriptor, uniform over the workgroup.
struct Tile {
  int gathered;  // 0: row r at position base + stride * r; 1: global column base + r
  int base;
  int stride;
  int count;     // rows >= count do not exist (their loads repeat a valid row; never attended)
  int ks0;       // kBand window tiles: residue-subsequence index of row 0
};

template <int D, int NW, int QB, int MODE>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int RW = 32 * QB;        // query rows per wave
  constexpr int QT = NW * RW;        // query rows per workgroup
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int KS = D / 16;         // MFMA k-steps over the head dim
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int MAT = kKeyTile * D * 2;
  constexpr int NLOAD = 2 * CH;      // 1 KB direct-load blocks per tile (K blocks, then V)
  constexpr int LPW = NLOAD / NW;    // of which each wave issues
  constexpr int RPB = 64 / CH;       // rows per 1 KB block
  constexpr int GREG = kGlobalCap / NT;
  static_assert(NLOAD % NW == 0, "direct-load blocks must split evenly over the waves");
  static_assert(kGlobalCap % NT == 0, "global staging must split evenly");
  constexpr bool kHasGlobalCols = MODE != kGlobalRows;

  __shared__ __attribute__((aligned(1024))) unsigned char st0[2 * MAT];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[2 * MAT];
  __shared__ int lay_list[MODE == kLayout ? 256 : 1];
  __shared__ int lay_cnt;
  __shared__ __attribute__((aligned(16))) int g_pos[kHasGlobalCols ? kGlobalCap : 1];
  __shared__ __attribute__((aligned(16))) int g_jr[kHasGlobalCols ? kGlobalCap : 1];
  __shared__ unsigned long long g_valid[kHasGlobalCols ? kGlobalCap / 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qj = lane & 31, hh = lane >> 5;

  // ------------------------------------------------------------------ work decomposition
  int b = 0, h = 0, dl = 1, p = 0, np = a.n, q0 = 0, ck = 0, rg = 0;
  if constexpr (MODE == kGlobalRows) {
    const int rgs = (a.g + QT - 1) / QT;
    int x = blockIdx.x;
    ck = x % a.chunks;
    x /= a.chunks;
    rg = x % rgs;
    x /= rgs;
    h = x % a.H;
    b = x / a.H;
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    b = L / a.tiles_per_b;
    int r = L - b * a.tiles_per_b;
    if (a.uniform_dil > 0) {
      const int tph = a.tile_off[1];
      h = r / tph;
      r -= h * tph;
      dl = a.uniform_dil;
    } else {
      int lo = 0, hi = a.H - 1;  // last head with tile_off[h] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.tile_off[mid] <= r) lo = mid; else hi = mid - 1;
      }
      h = lo;
      r -= a.tile_off[h];
      dl = a.dil[h];
    }
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
  const long bh = (long)b * a.H + h;
  const uint16_t* Qb = a.q + bh * a.n * D;
  const uint16_t* Kb = a.k + bh * a.n * D;
  const uint16_t* Vb = a.v + bh * a.n * D;
  const uint8_t* pad = a.kpad ? a.kpad + (long)b * a.n : nullptr;
  const int* gb = a.gidx ? a.gidx + (long)b * a.g : nullptr;

  // ------------------------------------------------------------------ query rows of this lane
  // Lane (qj, hh) holds query qb*32 + qj of the wave for every query block qb.
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
  u32x4 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[qb][s] = u32x4{0, 0, 0, 0};
      if (qpos[qb] >= 0)
        qf[qb][s] = *reinterpret_cast<const u32x4*>(Qb + (long)qpos[qb] * D + 16 * s + 8 * hh);
    }

  // kGlobalRows also publishes, once per (batch, global column), the column's position and
  // whether it is a usable key (in range, not padded) for the main kernel.
  if constexpr (MODE == kGlobalRows) {
    if (h == 0 && ck == 0 && hh == 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int c = rg * QT + wave * RW + 32 * qb + qj;
        if (c < a.g) {
          const int x = gb[c];
          const bool ok = x >= 0 && x < a.n && !(pad && pad[x]);
          a.gmeta[(long)b * a.g + c] = ok ? (int)(0x80000000u | (uint32_t)x) : 0;
        }
      }
    }
  }

  // ------------------------------------------------------------------ key tiles
  int n_local = 0, k_lo = 0, k_hi = -1, tpb = 1;
  if constexpr (MODE == kBand) {
    if (a.band_on) {
      const int q_last = min(q0 + QT, np) - 1;
      k_lo = max(0, q0 - a.wl);
      k_hi = min(np - 1, q_last + a.wr);
      n_local = (k_hi >= k_lo) ? (k_hi - k_lo + kKeyTile) / kKeyTile : 0;
    }
  } else if constexpr (MODE == kLayout) {
    tpb = a.block / kKeyTile;
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
    n_local = lay_cnt * tpb;
  } else {
    const int c0 = ck * kGlobalChunk;
    const int c1 = min(a.n, c0 + kGlobalChunk);
    n_local = (c1 > c0) ? (c1 - c0 + kKeyTile - 1) / kKeyTile : 0;
    k_lo = c0;
    k_hi = c1 - 1;
  }
  const int n_gtiles = (kHasGlobalCols && a.g > 0) ? (a.g + kKeyTile - 1) / kKeyTile : 0;
  const int n_tiles = n_local + n_gtiles;

  auto tile_of = [&](int t) -> Tile {
    Tile T;
    T.ks0 = 0;
    if (t >= n_local) {
      T.gathered = 1;
      T.base = (t - n_local) * kKeyTile;
      T.stride = 1;
      T.count = min(kKeyTile, a.g - T.base);
    } else if constexpr (MODE == kBand) {
      T.gathered = 0;
      T.ks0 = k_lo + t * kKeyTile;
      T.base = p + dl * T.ks0;
      T.stride = dl;
      T.count = min(kKeyTile, np - T.ks0);
    } else if constexpr (MODE == kLayout) {
      T.gathered = 0;
      T.base = lay_list[t / tpb] * a.block + (t % tpb) * kKeyTile;
      T.stride = 1;
      T.count = kKeyTile;
    } else {
      T.gathered = 0;
      T.base = k_lo + t * kKeyTile;
      T.stride = 1;
      T.count = min(kKeyTile, k_hi + 1 - T.base);
    }
    return T;
  };

  // ------------------------------------------------------------------ global columns
  // Positions, residue coordinates (for de-duplication against the window) and validity of
  // the global-key columns, staged once per workgroup in LDS.  The per-column records are
  // fetched at kernel start and written to LDS after the first tile's barrier.
  int gm_reg[GREG];
  if constexpr (kHasGlobalCols) {
#pragma unroll
    for (int i = 0; i < GREG; ++i) {
      const int c = tid + NT * i;
      gm_reg[i] = (n_gtiles > 0 && c < a.g) ? a.gmeta[(long)b * a.g + c] : 0;
    }
  }
  auto stage_globals = [&]() {
    if constexpr (kHasGlobalCols) {
#pragma unroll
      for (int i = 0; i < GREG; ++i) {
        const int c = tid + NT * i;
        const int m = gm_reg[i];
        bool ok = c < a.g && m < 0;  // bit 31: usable key
        const int pos = m & 0x7fffffff;
        if constexpr (MODE == kLayout) {
          const int blk = pos / a.block;
          for (int e = 0; e < lay_cnt; ++e) ok = ok && (lay_list[e] != blk);
        }
        int jr = kJrNone;
        if constexpr (MODE == kBand) {
          const int rel = pos - p;
          if (rel >= 0 && rel % dl == 0) jr = rel / dl;
        }
        g_pos[c] = pos;
        g_jr[c] = jr;
        const unsigned long long vm = __ballot(ok);
        if (lane == 0) g_valid[c >> 6] = vm;
      }
    }
  };

  // ------------------------------------------------------------------ tile loading
  // Block j of this wave covers rows RPB*sub .. RPB*sub + RPB - 1 of matrix `mat`; lane l writes
  // LDS bytes sub*1024 + 16*l, i.e. row RPB*sub + l/CH at swizzled chunk l%CH.
  // Row of tile and element offset of the 16-byte chunk that this lane moves in block j (kept as
  // a function of the lane, not in registers, to save VGPRs).
  auto ld_row = [&](int j) -> int { return ((wave * LPW + j) % CH) * RPB + lane / CH; };
  auto ld_col = [&](int j) -> int {
    const int blk = wave * LPW + j;
    const int row = ld_row(j);
    return 8 * ((lane % CH) ^ (blk / CH == 0 ? swz_k<D>(row) : swz_v<D>(row)));
  };
  auto issue = [&](unsigned char* st, const Tile& T) {
    int pos[LPW];
    if (kHasGlobalCols && T.gathered) {
#pragma unroll
      for (int j = 0; j < LPW; ++j) pos[j] = g_pos[T.base + min(ld_row(j), T.count - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < LPW; ++j) pos[j] = T.base + T.stride * min(ld_row(j), T.count - 1);
    }
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = wave * LPW + j;
      const int mat = blk / CH, sub = blk % CH;
      const uint16_t* src = (mat == 0 ? Kb : Vb) + ((long)pos[j] * D + ld_col(j));
      __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, st + mat * MAT + sub * 1024), 16, 0, 0);
    }
  };
  // key validity of a local tile: in range and (if padding is given) not padded; the pad byte of
  // row `lane` is loaded one tile ahead.  The load is issued on every path (from a harmless
  // address when there is no padding or no such row) so that the register is only ever written
  // by loads: overwriting it with a constant would force a wait for the loads in flight.
  auto pad_byte = [&](const Tile& T) -> int {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(Kb);
    if (pad && !T.gathered) src = pad + T.base + T.stride * min(lane, T.count - 1);
    return *src;
  };
  auto local_valid = [&](const Tile& T, int pb) -> unsigned long long {
    if (pad) return __ballot(lane < T.count && pb == 0);  // pb is a pad byte here
    return T.count >= 64 ? ~0ull : ((1ull << T.count) - 1ull);
  };

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
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 4 * db + 2 * (vg & 1) + ((vi & 3) >> 1);
    voff[db] = MAT + vrow0 * (2 * D) + ((chunk ^ vsw) * 16) + 8 * (vi & 1);
  }

  // ------------------------------------------------------------------ running state
  f32x16 o[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = neg_inf();
    l_run[qb] = 0.f;
  }
  const float c2 = a.scale_log2;

  // wave row range (kBand tile skipping)
  const int w_first = q0 + wave * RW;
  const int w_last = (MODE == kBand) ? min(w_first + RW - 1, np - 1) : w_first + RW - 1;
  bool wave_rows;
  if constexpr (MODE == kBand) wave_rows = w_first < np;
  else if constexpr (MODE == kLayout) wave_rows = true;
  else wave_rows = (rg * QT + wave * RW) < a.g;

  // ------------------------------------------------------------------ one tile
  // KIND 0: every key of the tile is allowed for every row of the wave (no masks);
  // KIND 1: per-element masks from the key validity bits and, in window mode, the band edges;
  // KIND 2: window mode global-key tile: validity bits plus removal of keys already attended
  //         through the window.
  // Each kind is compiled separately so the common interior tile carries no mask code.
  const uint32_t span = (uint32_t)(a.wl + a.wr);
  auto compute = [&](const unsigned char* st, const Tile& T, unsigned long long vmask,
                     bool need_band, auto kind_c) {
    constexpr int KIND = decltype(kind_c)::value;
    // The 64-key tile is processed as two 32-key halves kb: scores of half kb for every query
    // block, then the online-softmax step and the PV product of that half.  Keeping one half of
    // scores live at a time halves their registers; the scores MFMAs of half 1 can run under
    // the softmax VALU work of half 0.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // ---- scores S^T = K Q^T for keys 32kb..32kb+31
      f32x16 s[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(st + koff[ks] + kb * 32 * (2 * D));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = mfma_32x32x16(kf, qf[qb][ks], s[qb]);
      }

      // ---- masks.  Register r holds key 32kb + 8(r/4) + 4hh + r%4, i.e. bit 8(r/4) + r%4 of
      // w = (the tile's allowed keys for this lane's query) >> (32kb + 4hh).
      if constexpr (KIND == 2) {
        const uint32_t w = (uint32_t)(vmask >> (32 * kb + 4 * hh));
        const int* jr = g_jr + T.base + 32 * kb;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x4 jv = *reinterpret_cast<const u32x4*>(jr + 8 * g4 + 4 * hh);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = (w >> (8 * g4 + e)) & 1u;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              // a global key already inside this query's window is attended through the window
              const bool dup = (uint32_t)((int)jv[e] - (qsub[qb] - a.wl)) <= span;
              if (!ok || (a.band_on && dup)) s[qb][4 * g4 + e] = neg_inf();
            }
          }
        }
      } else if constexpr (KIND == 1) {
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
          const uint32_t w = (uint32_t)(m >> (32 * kb));
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) s[qb][r] = neg_inf();
        }
      }

      // ---- online softmax step in the log2 domain.  The running max is only raised when a
      // row's maximum exceeds it by more than 2^8; until then the stale max keeps every weight
      // below 2^8, which fp32 and bf16 hold without loss, and the final normalisation is exact.
      float xm[QB];
      bool need_any = false;
      bool need[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const f32x16& sv = s[qb];
        float x = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
        float y = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
        x = fmaxf(fmaxf(x, sv[6]), sv[7]);
        y = fmaxf(fmaxf(y, sv[8]), sv[9]);
        x = fmaxf(fmaxf(x, sv[10]), sv[11]);
        y = fmaxf(fmaxf(y, sv[12]), sv[13]);
        x = fmaxf(fmaxf(x, sv[14]), fmaxf(y, sv[15]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                         false, false);
        x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        xm[qb] = x;
        need[qb] = x > m_run[qb] && (m_run[qb] == neg_inf() || (x - m_run[qb]) * c2 > kRescaleLog2);
        need_any = need_any || need[qb];
      }
      if (__builtin_amdgcn_ballot_w64(need_any) != 0ull) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float alpha = need[qb] ? exp2_fast((m_run[qb] - xm[qb]) * c2) : 1.f;
          if (need[qb]) m_run[qb] = xm[qb];
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        }
      }

#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const f32x16& sv = s[qb];
        const float mc = (m_run[qb] == neg_inf()) ? 0.f : m_run[qb] * c2;
        uint32_t pk[8];
        float la = 0.f, lb = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float p0 = exp2_fast(__builtin_fmaf(sv[r], c2, -mc));
          const float p1 = exp2_fast(__builtin_fmaf(sv[r + 1], c2, -mc));
          const float p2 = exp2_fast(__builtin_fmaf(sv[r + 2], c2, -mc));
          const float p3 = exp2_fast(__builtin_fmaf(sv[r + 3], c2, -mc));
          pk[r >> 1] = pack_bf16x2(p0, p1);
          pk[(r >> 1) + 1] = pack_bf16x2(p2, p3);
          la += p0 + p1;
          lb += p2 + p3;
        }
        l_run[qb] += la + lb;

        // ---- O^T += V^T P^T for the two 16-key groups g = 2kb, 2kb+1 of this half
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
          const int g = 2 * kb + gh;
          const u32x4 bp = {pk[4 * gh + 0], pk[4 * gh + 1], pk[4 * gh + 2], pk[4 * gh + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const unsigned char* vp = st + voff[db] + 16 * g * (2 * D);
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp));
            const s16x4 v1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vp + 8 * (2 * D)));
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
            o[qb][db] = mfma_32x32x16(va, bp, o[qb][db]);
          }
        }
      }
    }
  };
  auto compute_tile = [&](const unsigned char* st, const Tile& T, unsigned long long vmask) {
    bool need_band = false;
    if constexpr (MODE == kBand) {
      if (!T.gathered) {
        const int kf = T.ks0, kl = T.ks0 + kKeyTile - 1;
        if (kl < w_first - a.wl || kf > w_last + a.wr) return;  // no key of the tile in reach
        need_band = !(kf >= w_last - a.wl && kl <= w_first + a.wr);
      }
      if (T.gathered) {
        compute(st, T, vmask, false, std::integral_constant<int, 2>{});
        return;
      }
    }
    if (need_band || vmask != ~0ull) compute(st, T, vmask, need_band, std::integral_constant<int, 1>{});
    else compute(st, T, vmask, false, std::integral_constant<int, 0>{});
  };

  // ------------------------------------------------------------------ tile loop
  // Two LDS stages: tile t computes from stage t%2 while tile t+1 streams into the other.  The
  // barrier at the top of each step (it waits for this wave's outstanding loads first) makes
  // tile t visible to every wave and retires every read of the stage about to be refilled.
  if (n_tiles > 0) {
    if (n_local == 0) {
      stage_globals();
      __syncthreads();
    }
    int pb_next = 0;
    {
      const Tile T0 = tile_of(0);
      issue(st0, T0);
      pb_next = pad_byte(T0);
    }
    // One step: wait for tile t (this wave's loads, then the barrier for everyone's), start
    // tile t+1 into the other stage, compute tile t.  The loop is unrolled by two so that the
    // stage being read and the stage being filled are distinct arrays at compile time; with a
    // run-time choice the compiler must assume they alias and would wait for the new loads
    // before every LDS read.
    auto step = [&](unsigned char* cur, unsigned char* nxt, int t) {
      wait_loads_then_barrier();
      const Tile T = tile_of(t);
      unsigned long long vmask;
      if constexpr (kHasGlobalCols) {
        vmask = T.gathered ? g_valid[T.base >> 6] : local_valid(T, pb_next);
      } else {
        vmask = local_valid(T, pb_next);
      }
      if (t == 0 && n_local > 0 && n_gtiles > 0) {
        stage_globals();
        if (n_local == 1) __syncthreads();
      }
      if (t + 1 < n_tiles) {
        const Tile Tn = tile_of(t + 1);
        issue(nxt, Tn);
        pb_next = pad_byte(Tn);
      }
      if (wave_rows) compute_tile(cur, T, vmask);
    };
    for (int t = 0; t < n_tiles; t += 2) {
      step(st0, st1, t);
      if (t + 1 < n_tiles) step(st1, st0, t + 1);
    }
  }

  // ------------------------------------------------------------------ epilogue
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __uint_as_float(__shfl_xor(__float_as_uint(l_run[qb]), 32));
    if constexpr (MODE == kGlobalRows) {
      if (qpos[qb] >= 0) {
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
          pml[0] = (m_run[qb] == neg_inf()) ? neg_inf() : m_run[qb] * c2;
          pml[1] = l_tot;
        }
      }
    } else {
      if (qpos[qb] < 0) continue;
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      uint16_t* orow = a.out + (bh * a.n + qpos[qb]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + 4 * hh;
          u32x2 w;
          w[0] = pack_bf16x2(o[qb][db][4 * rq] * inv, o[qb][db][4 * rq + 1] * inv);
          w[1] = pack_bf16x2(o[qb][db][4 * rq + 2] * inv, o[qb][db][4 * rq + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d) = w;
        }
      if (a.lse && hh == 0)
        a.lse[bh * a.n + qpos[qb]] =
            (l_tot > 0.f) ? (m_run[qb] * c2 + __log2f(l_tot)) * kLn2 : neg_inf();
    }
  }
}

// Merge the per-chunk partials of every global row and write its output and lse.
// One wave per (batch, head, global row); each lane owns D/64 output columns.
template <int D>
__global__ __launch_bounds__(64) void global_combine_kernel(FwdArgs a) {
  const int lane = threadIdx.x;
  const long row = blockIdx.x;  // (b*H + h)*g + c
  const long bh = row / a.g;
  const int c = (int)(row % a.g);
  const int b = (int)(bh / a.H);
  const int pos = a.gidx[(long)b * a.g + c];
  if (pos < 0 || pos >= a.n) return;  // out-of-range global index: nothing to write
  const float* po = a.part + row * a.chunks * D;
  const float* pml = a.part + (long)a.B * a.H * a.g * a.chunks * D + row * a.chunks * 2;
  // each lane holds the (m, l) of chunks lane, lane + 64, ...
  float M = -__builtin_inff();
  for (int k = lane; k < a.chunks; k += 64) M = fmaxf(M, pml[2 * k]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int k0 = 0; k0 < a.chunks; k0 += 64) {
      const int k = k0 + lane;
      float w = 0.f, lk = 0.f;
      if (k < a.chunks) {
        const float mk = pml[2 * k];
        if (mk != -__builtin_inff()) {
          w = exp2f(mk - M);
          lk = pml[2 * k + 1];
        }
      }
      L += w * lk;
      const int kn = min(64, a.chunks - k0);
      for (int kk = 0; kk < kn; ++kk) {
        const float wk = __shfl(w, kk);
        if (wk == 0.f) continue;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += wk * po[(long)(k0 + kk) * D + lane + 64 * e];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint16_t* orow = a.out + (bh * a.n + pos) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float v = acc[e] * inv;
    orow[lane + 64 * e] = __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  if (a.lse && lane == 0)
    a.lse[bh * a.n + pos] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

template <int D, int NW, int QB, int MODE>
hipError_t launch_one(const FwdArgs& a, long grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, MODE>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

// Query rows per workgroup of the main kernel: 128 in window mode, the block size in layout mode.
int main_rows_per_workgroup(int mode, int block) { return mode == kLayout ? block : 128; }

hipError_t launch_mfma_main(const FwdArgs& a, int d, int mode, int grid, hipStream_t s) {
  if (mode == kBand) {
    if (d == 64) return launch_one<64, 4, 1, kBand>(a, grid, s);
    if (d == 128) return launch_one<128, 4, 1, kBand>(a, grid, s);
  } else if (mode == kLayout) {
    if (a.block == 64) {
      if (d == 64) return launch_one<64, 2, 1, kLayout>(a, grid, s);
      if (d == 128) return launch_one<128, 2, 1, kLayout>(a, grid, s);
    } else if (a.block == 128) {
      if (d == 64) return launch_one<64, 2, 2, kLayout>(a, grid, s);
      if (d == 128) return launch_one<128, 4, 1, kLayout>(a, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

int global_rows_per_workgroup(int g) { return g <= 64 ? 64 : 128; }

hipError_t launch_mfma_global_partial(const FwdArgs& a, int d, hipStream_t s) {
  const int qt = global_rows_per_workgroup(a.g);
  const long grid = (long)a.B * a.H * ((a.g + qt - 1) / qt) * a.chunks;
  if (qt == 64) {
    if (d == 64) return launch_one<64, 2, 1, kGlobalRows>(a, grid, s);
    if (d == 128) return launch_one<128, 2, 1, kGlobalRows>(a, grid, s);
  } else {
    if (d == 64) return launch_one<64, 2, 2, kGlobalRows>(a, grid, s);
    if (d == 128) return launch_one<128, 4, 1, kGlobalRows>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_global_combine(const FwdArgs& a, int d, hipStream_t s) {
  const long grid = (long)a.B * a.H * a.g;
  if (grid <= 0) return hipSuccess;
  if (d == 64) hipLaunchKernelGGL(global_combine_kernel<64>, dim3(grid), dim3(64), 0, s, a);
  else if (d == 128) hipLaunchKernelGGL(global_combine_kernel<128>, dim3(grid), dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace longattn
