// bf16 sparse attention forward on gfx950 matrix cores.
//
// One kernel template serves three workgroup kinds:
//   kBand        query tile of 32*NW rows of one (batch, head, dilation residue); walks the key
//                tiles that intersect the window, then the global-key columns.
//   kLayout      one query block of a block-sparse layout; walks the listed key blocks, then the
//                global-key columns.
//   kGlobalRows  up to 32*NW global query rows against one chunk of keys; writes unnormalised
//                partial results that the combine kernel merges.
//
// Attention over a key set is exact masked softmax attention: the window, the global tokens and
// the layout blocks are a set of allowed (query, key) edges, each counted once (Big Bird reading
// notes, sections 3.1 and 3.3).  A dilated window is split into dil independent undilated windows
// over the residue classes i = p (mod dil) (the window skips tokens like a dilated convolution,
// Longformer hub page, section 2), so every tile here is a plain contiguous or strided band.
// Global-key columns are concatenated after the local keys and share one online softmax with
// them, as the LongT5 guide describes for its side keys (blocking-helpers paragraph).
//
// Wave-level math (32x32x16 bf16 MFMA, fp32 accumulate).  Each wave owns 32 query rows and
// computes the transposed score block S^T = K Q^T, so every lane holds the scores of exactly one
// query (its column) for 32 of the 64 keys of a tile; the other 32 sit in lane ^ 32.  Row max and
// row sum are therefore in-lane reductions plus one exchange with lane ^ 32.  The output is kept
// transposed as well, O^T += V^T P^T, so the softmax rescale factor is per lane.  V is written to
// LDS transposed (with the key order inside each group of 16 permuted) so that every A operand
// of both products is one 16-byte LDS read.

#include "attn_args.h"

namespace longattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kJrNone = -(1 << 29);  // "this global key is not in the query's residue class"

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

// Logical workgroup id such that consecutive ids run on the same XCD.  Workgroups are handed to
// the 8 XCDs round robin, so neighbouring query tiles (which re-read the same K/V rows) would
// otherwise land in 8 different L2 caches.  This is a bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int x, int G) {
  const int q = G >> 3, r = G & 7;
  const int xcd = x & 7, idx = x >> 3;
  return xcd * q + min(xcd, r) + idx;
}

// Key tile descriptor, uniform over the workgroup.
struct Tile {
  int gathered;  // 0: row r is at position base + stride * r; 1: global column base + r
  int base;
  int stride;
  int count;     // rows r >= count do not exist (loaded as zeros, never valid)
  int ks0;       // kBand local tiles: residue-subsequence index of row 0
};

template <int D, int NW, int MODE>
struct Smem {
  static constexpr int kMatBytes = kKeyTile * D * 2;           // one K tile or one V^T tile
  static constexpr int kMetaBytes = 8 + 8 + 4 * kKeyTile;        // valid mask, pad, jr[64]
  static constexpr int kStageBytes = 2 * kMatBytes + kMetaBytes;
  static constexpr int kListInts = 256;                          // compacted layout row
  static constexpr int kBytes = 2 * kStageBytes + 4 * kListInts + 16;
};

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int QT = NW * 32;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;        // 16-byte chunks per row of K
  constexpr int TASKS = 4 * D;     // (4 rows x 1 chunk) load tasks: 2D for K, 2D for V
  constexpr int TPT = (TASKS + NT - 1) / NT;
  using S = Smem<D, NW, MODE>;
  static_assert(TASKS % NT == 0, "load tasks must divide evenly");

  __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
  int* list = reinterpret_cast<int*>(smem + 2 * S::kStageBytes);
  int* list_count = list + S::kListInts;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qj = lane & 31, hh = lane >> 5;

  // ------------------------------------------------------------------ work decomposition
  int b = 0, h = 0, dl = 1, p = 0, np = a.n, q0 = 0, ck = 0, rg = 0;
  if (MODE == kGlobalRows) {
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
    if (MODE == kBand) {
      for (;;) {  // residue class p holds ceil((n - p) / dl) positions
        const int n_p = (a.n - p + dl - 1) / dl;
        const int t_p = (n_p + QT - 1) / QT;
        if (r < t_p) { np = n_p; break; }
        r -= t_p;
        ++p;
      }
      q0 = r * QT;
    } else {
      q0 = r * a.block;  // kLayout: query block r, QT == block
    }
  }
  const long bh = (long)b * a.H + h;
  const uint16_t* Qb = a.q + bh * a.n * D;
  const uint16_t* Kb = a.k + bh * a.n * D;
  const uint16_t* Vb = a.v + bh * a.n * D;
  const uint8_t* pad = a.kpad ? a.kpad + (long)b * a.n : nullptr;
  const int* gb = a.gidx ? a.gidx + (long)b * a.g : nullptr;

  // ------------------------------------------------------------------ key tiles
  int n_local = 0, k_lo = 0, k_hi = -1, tpb = 1;
  if (MODE == kBand) {
    if (a.band_on) {
      const int q_last = min(q0 + QT, np) - 1;
      k_lo = max(0, q0 - a.wl);
      k_hi = min(np - 1, q_last + a.wr);
      n_local = (k_hi >= k_lo) ? (k_hi - k_lo + kKeyTile) / kKeyTile : 0;
    }
  } else if (MODE == kLayout) {
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
        if (id >= 0) list[base + __popcll(m & ((1ull << lane) - 1ull))] = id;
        base += __popcll(m);
      }
      if (lane == 0) *list_count = base;
    }
    __syncthreads();
    n_local = *list_count * tpb;
  } else {
    const int c0 = ck * kGlobalChunk;
    const int c1 = min(a.n, c0 + kGlobalChunk);
    n_local = (c1 > c0) ? (c1 - c0 + kKeyTile - 1) / kKeyTile : 0;
    k_lo = c0;
    k_hi = c1 - 1;
  }
  const int n_gtiles = (MODE != kGlobalRows && a.g > 0) ? (a.g + kKeyTile - 1) / kKeyTile : 0;
  const int n_tiles = n_local + n_gtiles;

  auto tile_of = [&](int t) -> Tile {
    Tile T;
    T.ks0 = 0;
    if (t >= n_local) {
      T.gathered = 1;
      T.base = (t - n_local) * kKeyTile;
      T.stride = 1;
      T.count = min(kKeyTile, a.g - T.base);
    } else if (MODE == kBand) {
      T.gathered = 0;
      T.ks0 = k_lo + t * kKeyTile;
      T.base = p + dl * T.ks0;
      T.stride = dl;
      T.count = min(kKeyTile, np - T.ks0);
    } else if (MODE == kLayout) {
      T.gathered = 0;
      T.base = list[t / tpb] * a.block + (t % tpb) * kKeyTile;
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

  // ------------------------------------------------------------------ query rows of this lane
  const int qrow = wave * 32 + qj;  // row inside the workgroup tile
  int qpos = -1;                    // sequence position, -1 = no such row
  int qs = 0;                       // kBand: residue-subsequence index
  if (MODE == kBand) {
    qs = q0 + qrow;
    if (qs < np) qpos = p + dl * qs;
  } else if (MODE == kLayout) {
    qpos = q0 + qrow;
  } else {
    const int c = rg * QT + qrow;
    if (c < a.g) qpos = gb[c];
    if (qpos >= a.n) qpos = -1;
  }
  // wave row range (for tile skipping), kBand only
  const int w_first = q0 + wave * 32;
  const int w_last = min(q0 + wave * 32 + 31, np - 1);
  bool wave_rows;
  if (MODE == kBand) wave_rows = w_first < np;
  else if (MODE == kLayout) wave_rows = true;
  else wave_rows = (rg * QT + wave * 32) < a.g;

  u32x4 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    qf[s] = u32x4{0, 0, 0, 0};
    if (qpos >= 0)
      qf[s] = *reinterpret_cast<const u32x4*>(Qb + (long)qpos * D + 16 * s + 8 * hh);
  }

  // ------------------------------------------------------------------ tile loading
  // Task tk < 2D: K rows 4*rq..4*rq+3, chunk c.  Task tk >= 2D: the same for V.
  u32x4 stage_regs[TPT][4];
  int meta_pos = -1;
  bool meta_ok = false;

  auto issue_loads = [&](const Tile& T) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int tk = tid + u * NT;
      const bool isv = tk >= 2 * D;
      const int t2 = isv ? tk - 2 * D : tk;
      const int rq = t2 / CH, c = t2 % CH;
      const uint16_t* src = isv ? Vb : Kb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rq + i;
        int pos = -1;
        if (r < T.count) pos = T.gathered ? gb[T.base + r] : T.base + T.stride * r;
        if (pos >= a.n) pos = -1;
        stage_regs[u][i] = u32x4{0, 0, 0, 0};
        if (pos >= 0) stage_regs[u][i] = *reinterpret_cast<const u32x4*>(src + (long)pos * D + 8 * c);
      }
    }
    if (wave == 0) {  // key validity of row `lane`
      meta_pos = -1;
      meta_ok = false;
      if (lane < T.count) {
        meta_pos = T.gathered ? gb[T.base + lane] : T.base + T.stride * lane;
        if (meta_pos < 0 || meta_pos >= a.n) meta_pos = -1;
        meta_ok = meta_pos >= 0 && !(pad && pad[meta_pos]);
        if (MODE == kLayout && T.gathered) {  // already attended through a layout block?
          const int blk = meta_pos / a.block;
          const int cnt = *list_count;
          for (int e = 0; e < cnt; ++e) meta_ok = meta_ok && (list[e] != blk);
        }
      }
    }
  };

  auto store_stage = [&](int st, const Tile& T) {
    unsigned char* base = smem + st * S::kStageBytes;
    unsigned char* kt = base;
    unsigned char* vt = base + S::kMatBytes;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int tk = tid + u * NT;
      const bool isv = tk >= 2 * D;
      const int t2 = isv ? tk - 2 * D : tk;
      const int rq = t2 / CH, c = t2 % CH;
      if (!isv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * rq + i;
          const int phys = c ^ (r & 7);
          *reinterpret_cast<u32x4*>(kt + r * (D * 2) + phys * 16) = stage_regs[u][i];
        }
      } else {
        // rows = keys 4rq..4rq+3, columns = d 8c..8c+7: write V^T[d][keys] (8 bytes per d)
        const int G = rq >> 2, qg = rq & 3;
        const int chunk = 2 * G + (qg & 1);
        const int boff = 8 * (qg >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * c + e;
          const int wsel = e >> 1;
          uint32_t x0 = stage_regs[u][0][wsel], x1 = stage_regs[u][1][wsel];
          uint32_t x2 = stage_regs[u][2][wsel], x3 = stage_regs[u][3][wsel];
          u32x2 w;
          if (e & 1) {
            w[0] = (x0 >> 16) | (x1 & 0xFFFF0000u);
            w[1] = (x2 >> 16) | (x3 & 0xFFFF0000u);
          } else {
            w[0] = (x0 & 0xFFFFu) | (x1 << 16);
            w[1] = (x2 & 0xFFFFu) | (x3 << 16);
          }
          const int phys = chunk ^ (d & 7);
          *reinterpret_cast<u32x2*>(vt + d * 128 + phys * 16 + boff) = w;
        }
      }
    }
    if (wave == 0) {
      const unsigned long long vm = __ballot(meta_ok);
      unsigned char* meta = base + 2 * S::kMatBytes;
      if (lane == 0) *reinterpret_cast<unsigned long long*>(meta) = vm;
      if (MODE == kBand) {
        int jr = kJrNone;
        if (meta_pos >= 0 && T.gathered) {
          const int rel = meta_pos - p;
          if (rel >= 0 && rel % dl == 0) jr = rel / dl;
        }
        reinterpret_cast<int*>(meta + 16)[lane] = jr;
      }
    }
  };

  // ------------------------------------------------------------------ running state
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = neg_inf();
  float l_run = 0.f;
  const float c2 = a.scale_log2;

  if (n_tiles > 0) {
    Tile T0 = tile_of(0);
    issue_loads(T0);
    store_stage(0, T0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int st = t & 1;
    const Tile T = tile_of(t);
    Tile Tn;
    const bool has_next = (t + 1) < n_tiles;
    if (has_next) {
      Tn = tile_of(t + 1);
      issue_loads(Tn);
    }

    // ---- does this wave need the tile, and which masks apply?
    bool active = wave_rows;
    bool need_band = false;
    if (MODE == kBand && !T.gathered) {
      const int kf = T.ks0, kl = T.ks0 + kKeyTile - 1;
      if (kl < w_first - a.wl || kf > w_last + a.wr) active = false;
      need_band = !(kf >= w_last - a.wl && kl <= w_first + a.wr);
    }
    const unsigned char* base = smem + st * S::kStageBytes;
    const unsigned char* meta = base + 2 * S::kMatBytes;
    const unsigned long long vmask = *reinterpret_cast<const unsigned long long*>(meta);

    if (active) {
      const unsigned char* kt = base;
      const unsigned char* vt = base + S::kMatBytes;
      // ---- scores S^T = K Q^T for keys 0-31 (s0) and 32-63 (s1)
      f32x16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int c = 2 * s + hh;
        const int r0 = qj, r1 = 32 + qj;
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(kt + r0 * (D * 2) + ((c ^ (r0 & 7)) * 16));
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(kt + r1 * (D * 2) + ((c ^ (r1 & 7)) * 16));
        s0 = mfma_32x32x16(k0, qf[s], s0);
        s1 = mfma_32x32x16(k1, qf[s], s1);
      }

      // ---- masks.  Register r of block kb holds key 32*kb + 8*(r/4) + 4*hh + r%4.
      const bool need_keys = vmask != ~0ull;
      if (T.gathered && MODE == kBand) {
        const int* jr = reinterpret_cast<const int*>(meta + 16);
        const uint32_t lo_w = (uint32_t)(vmask >> (4 * hh));
        const uint32_t hi_w = (uint32_t)(vmask >> (32 + 4 * hh));
        const int rel0 = qs - a.wl;
        const uint32_t span = (uint32_t)(a.wl + a.wr);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x4 j0 = *reinterpret_cast<const u32x4*>(jr + 8 * g4 + 4 * hh);
          const u32x4 j1 = *reinterpret_cast<const u32x4*>(jr + 32 + 8 * g4 + 4 * hh);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            const int cb = 8 * g4 + e;
            const bool in0 = a.band_on && ((uint32_t)((int)j0[e] - rel0) <= span);
            const bool in1 = a.band_on && ((uint32_t)((int)j1[e] - rel0) <= span);
            if (!((lo_w >> cb) & 1u) || in0) s0[r] = neg_inf();
            if (!((hi_w >> cb) & 1u) || in1) s1[r] = neg_inf();
          }
        }
      } else if (need_band || need_keys) {
        unsigned long long m = vmask >> (4 * hh);
        if (need_band) {
          // keys k with qs - wl <= ks0 + k <= qs + wr, shifted by this lane's 4*hh
          const int lo = qs - a.wl - T.ks0 - 4 * hh;
          const int hi = qs + a.wr - T.ks0 - 4 * hh;
          unsigned long long bm = 0ull;
          if (hi >= 0 && lo <= 63) {
            const int lc = max(lo, 0), hc = min(hi, 63);
            bm = (~0ull >> (63 - (hc - lc))) << lc;
          }
          m &= bm;
        }
        const uint32_t lo_w = (uint32_t)m, hi_w = (uint32_t)(m >> 32);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cb = 8 * (r >> 2) + (r & 3);
          if (!((lo_w >> cb) & 1u)) s0[r] = neg_inf();
          if (!((hi_w >> cb) & 1u)) s1[r] = neg_inf();
        }
      }

      // ---- online softmax (log2 domain; scores scaled inside the exponent)
      float mx = neg_inf();
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float mc = (m_new == neg_inf()) ? 0.f : m_new * c2;
      const float alpha = exp2_fast(m_run * c2 - mc);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

      uint32_t pk[2][8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p00 = exp2_fast(__builtin_fmaf(s0[r], c2, -mc));
        const float p01 = exp2_fast(__builtin_fmaf(s0[r + 1], c2, -mc));
        const float p10 = exp2_fast(__builtin_fmaf(s1[r], c2, -mc));
        const float p11 = exp2_fast(__builtin_fmaf(s1[r + 1], c2, -mc));
        l_run += (p00 + p01) + (p10 + p11);
        pk[0][r >> 1] = pack_bf16x2(p00, p01);
        pk[1][r >> 1] = pack_bf16x2(p10, p11);
      }

      // ---- O^T += V^T P^T, four groups of 16 keys
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 bp = {pk[g >> 1][4 * (g & 1) + 0], pk[g >> 1][4 * (g & 1) + 1],
                          pk[g >> 1][4 * (g & 1) + 2], pk[g >> 1][4 * (g & 1) + 3]};
        const int c = 2 * g + hh;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = 32 * db + qj;
          const u32x4 av = *reinterpret_cast<const u32x4*>(vt + d * 128 + ((c ^ (d & 7)) * 16));
          o[db] = mfma_32x32x16(av, bp, o[db]);
        }
      }
    }

    if (has_next) store_stage(st ^ 1, Tn);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (MODE == kGlobalRows) {
    if (qpos >= 0) {
      const int c = rg * QT + qrow;
      const long slot = (bh * a.g + c) * a.chunks + ck;
      float* po = a.part + slot * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + 4 * hh;
          *reinterpret_cast<float4*>(po + d) =
              make_float4(o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]);
        }
      if (hh == 0) {
        float* pml = a.part + (long)a.B * a.H * a.g * a.chunks * D + slot * 2;
        pml[0] = (m_run == neg_inf()) ? neg_inf() : m_run * c2;
        pml[1] = l_tot;
      }
    }
    return;
  }
  if (qpos < 0) return;
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
    a.lse[bh * a.n + qpos] = (l_tot > 0.f) ? (m_run * c2 + __log2f(l_tot)) * kLn2 : neg_inf();
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
  float M = -__builtin_inff();
  for (int k = 0; k < a.chunks; ++k) M = fmaxf(M, pml[2 * k]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int k = 0; k < a.chunks; ++k) {
      const float mk = pml[2 * k];
      if (mk == -__builtin_inff()) continue;
      const float w = exp2f(mk - M);
      L += w * pml[2 * k + 1];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * po[(long)k * D + lane + 64 * e];
    }
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

template <int D, int NW, int MODE>
hipError_t launch_one(const FwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, NW, MODE>), dim3(grid), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_main(const FwdArgs& a, int d, int mode, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (mode == kBand) {
    if (d == 64) return launch_one<64, 4, kBand>(a, grid, s);
    if (d == 128) return launch_one<128, 4, kBand>(a, grid, s);
  } else if (mode == kLayout) {
    if (a.block == 64) {
      if (d == 64) return launch_one<64, 2, kLayout>(a, grid, s);
      if (d == 128) return launch_one<128, 2, kLayout>(a, grid, s);
    } else if (a.block == 128) {
      if (d == 64) return launch_one<64, 4, kLayout>(a, grid, s);
      if (d == 128) return launch_one<128, 4, kLayout>(a, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_global_partial(const FwdArgs& a, int d, int nw, hipStream_t s) {
  const int qt = nw * 32;
  const long grid = (long)a.B * a.H * ((a.g + qt - 1) / qt) * a.chunks;
  if (grid <= 0) return hipSuccess;
  if (nw == 1) {
    if (d == 64) return launch_one<64, 1, kGlobalRows>(a, (int)grid, s);
    if (d == 128) return launch_one<128, 1, kGlobalRows>(a, (int)grid, s);
  } else if (nw == 2) {
    if (d == 64) return launch_one<64, 2, kGlobalRows>(a, (int)grid, s);
    if (d == 128) return launch_one<128, 2, kGlobalRows>(a, (int)grid, s);
  } else if (nw == 4) {
    if (d == 64) return launch_one<64, 4, kGlobalRows>(a, (int)grid, s);
    if (d == 128) return launch_one<128, 4, kGlobalRows>(a, (int)grid, s);
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
