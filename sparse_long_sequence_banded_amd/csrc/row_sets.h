// Key sets of single query rows and query sets of single key columns, for the per-row kernels
// (fp32 forward, entry counter, and the backward passes of every pattern).
//
// Rows walk their candidate keys in this order, keeping a candidate only if it is not padded and
// was not listed earlier:
//   global row:     every position (a global token attends the whole sequence; Longformer hub
//                   page, section 2; Big Bird reading notes, section 3.2.3);
//   any other row:  the window keys i + dil*t, t in [-win_left, win_right], inside [0, n)
//                   (Big Bird notes, section 3.2.1; dilation as on the Longformer hub page,
//                   section 2), then the global tokens, then the keys of the listed layout
//                   blocks (Big Bird notes, sections 3.2.2 and 3.3).
// Duplicates are dropped by testing membership in the earlier sets, so each (query, key) edge is
// counted once, as in the graph view of sparse attention (Big Bird notes, section 3.1).
//
// Columns (the query rows that attend key j, for the key-side gradients) list the same edges
// from the other end: none if j is padded; every row if j is a global token; otherwise the global
// rows, then the window rows j - dil*t, t in [-win_left, win_right], inside [0, n) and not global,
// then the rows of every query block whose layout lists j's block that are neither global nor in
// the window.
#pragma once

#include "attn_args.h"

namespace longattn {
namespace rowsets {

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

__device__ inline RowCtx make_row(const FwdArgs& a, long row) {
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
__device__ inline int candidate_key(const FwdArgs& a, const RowCtx& r, long c) {
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


// ---------------------------------------------------------------------------- key columns
struct ColCtx {
  int b, h, j, dl;
  bool padded, is_global;
  int t_lo, n_band;  // window rows j - dl * (t_lo + c), c < n_band
  const int* gb;
};

__device__ inline ColCtx make_col(const FwdArgs& a, long col) {
  ColCtx c;
  c.j = (int)(col % a.n);
  const long bh = col / a.n;
  c.h = (int)(bh % a.H);
  c.b = (int)(bh / a.H);
  c.dl = a.uniform_dil > 0 ? a.uniform_dil : a.dil[c.h];
  c.gb = a.gidx ? a.gidx + (long)c.b * a.g : nullptr;
  c.padded = a.kpad && a.kpad[(long)c.b * a.n + c.j];
  c.is_global = a.g > 0 && sorted_contains(c.gb, a.g, c.j);
  c.t_lo = 0;
  c.n_band = 0;
  if (a.band_on) {
    // rows i = j - dl*t inside [0, n): t <= j/dl and t >= -(n-1-j)/dl
    const int t_lo = max(-a.wl, -floor_div(a.n - 1 - c.j, c.dl));
    const int t_hi = min(a.wr, floor_div(c.j, c.dl));
    c.t_lo = t_lo;
    c.n_band = max(0, t_hi - t_lo + 1);
  }
  return c;
}

// Whether the layout row of query block qb (head h) lists key block kb.
__device__ inline bool layout_lists(const FwdArgs& a, int h, int qb, int kb) {
  const int nb = a.n / a.block;
  const int* row = a.layout + ((long)h * nb + qb) * a.max_kb;
  for (int s = 0; s < a.max_kb; ++s)
    if (row[s] == kb) return true;
  return false;
}

// Window row of candidate c (c < n_band), or -1 if it is a global row (listed already).
__device__ inline int column_band_row(const FwdArgs& a, const ColCtx& c, int idx) {
  const int i = c.j - c.dl * (c.t_lo + idx);
  if (a.g > 0 && sorted_contains(c.gb, a.g, i)) return -1;
  return i;
}

// Layout row i (of a block that lists j's block) unless it is global or already a window row.
__device__ inline bool column_layout_row_ok(const FwdArgs& a, const ColCtx& c, int i) {
  if (a.g > 0 && sorted_contains(c.gb, a.g, i)) return false;
  if (a.band_on) {
    const long dd = (long)c.j - i;
    if (dd % c.dl == 0) {
      const long t = dd / c.dl;
      if (t >= -a.wl && t <= a.wr) return false;
    }
  }
  return true;
}

}  // namespace rowsets
}  // namespace longattn
