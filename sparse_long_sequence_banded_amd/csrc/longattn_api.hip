// C-ABI boundary: argument validation, planning and kernel dispatch.
//
// Nothing here computes attention; every arithmetic step runs in the kernels of attn_mfma.hip
// (bf16) and attn_rowwise.hip (fp32 and the entry counter).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "attn_args.h"
#include "longattn.h"

using namespace longattn;

namespace {

constexpr long kMaxElems = 1L << 46;        // B*H*n*d bound for 64-bit offset arithmetic
constexpr int kMaxN = 1 << 28;              // keeps every position and sentinel in int32

struct Plan {
  FwdArgs a;
  bool bf16 = false;
  int mode = kBand;
  long grid_main = 0;
  size_t part_floats = 0;
  size_t ws_bytes = 0;
  bool empty = false;
};

bool debug_enabled() {
  const char* e = std::getenv("LONGATTN_DEBUG");
  return e && e[0] == '1';
}

// Keys per global-row partial workgroup of the forward pass (rows per global-owner workgroup of
// the backward): 512.  Those workgroups are dispatched after all the main ones, so they fill the
// last round as main workgroups finish, and shorter ones fill it more evenly.  Forward, window
// mode, 512 keys against 1024: the attention kernel 4.7% faster on the 16K dilated workload and
// 8.6% on the 4K one, for 0.5 us more in the combine (384, 640 and 768 fell in between; a 64-row
// block layout: 7% faster).  Backward, 512 rows with the owners last against 1024 first: the 4K
// window workload 11% and the 4K block layout 16% faster, the 16K ones unchanged (256 and 384:
// slower).
int forward_chunk_keys(const longattn_desc* d) {
  (void)d;
  return kGlobalChunk;
}

longattn_status plan_call(const longattn_desc* d, bool for_forward, Plan* P,
                          int chunk_keys = kGlobalChunk) {
  if (!d) return LONGATTN_ERR_INVALID_ARG;
  if (d->batch < 0 || d->heads < 0 || d->n < 0 || d->d < 1) return LONGATTN_ERR_INVALID_ARG;
  if (d->dtype != LONGATTN_BF16 && d->dtype != LONGATTN_F32) return LONGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(d->scale) || !(d->scale > 0.f)) return LONGATTN_ERR_INVALID_ARG;
  const bool band_off = d->win_left == -1 && d->win_right == -1;
  if (!band_off && (d->win_left < 0 || d->win_right < 0)) return LONGATTN_ERR_INVALID_ARG;
  if (d->n_global < 0 || d->n_global > d->n) return LONGATTN_ERR_INVALID_ARG;
  if (d->n_global > 0 && !d->global_idx) return LONGATTN_ERR_INVALID_ARG;
  if (d->block_layout) {
    if (d->block < 1 || d->max_kb < 0 || (d->n % d->block) != 0) return LONGATTN_ERR_INVALID_ARG;
  }
  if (d->dilation) {
    for (int h = 0; h < d->heads; ++h)
      if (d->dilation[h] < 1) return LONGATTN_ERR_INVALID_ARG;
  }
  if (d->n > kMaxN) return LONGATTN_ERR_UNSUPPORTED;
  {
    long e = 1;
    const long dims[4] = {d->batch, d->heads, d->n, d->d};
    for (long x : dims) {
      if (x == 0) { e = 0; break; }
      if (e > kMaxElems / x) return LONGATTN_ERR_UNSUPPORTED;
      e *= x;
    }
  }

  Plan& p = *P;
  p = Plan();
  FwdArgs& a = p.a;
  std::memset(&a, 0, sizeof(a));
  p.bf16 = d->dtype == LONGATTN_BF16;
  const bool has_layout = d->block_layout != nullptr;

  if (for_forward) {
    if (p.bf16) {
      if (d->d != 64 && d->d != 128) return LONGATTN_ERR_UNSUPPORTED;
      // per-head K/V byte offsets are 32-bit buffer offsets in the kernels
      if ((long)d->n * d->d * 2 > 0x7fffffffL) return LONGATTN_ERR_UNSUPPORTED;
      if (has_layout && !band_off) return LONGATTN_ERR_UNSUPPORTED;
      if (has_layout && ((d->block != 64 && d->block != 128) || d->max_kb > 256))
        return LONGATTN_ERR_UNSUPPORTED;
      if (d->n_global > kGlobalCap) return LONGATTN_ERR_UNSUPPORTED;
    } else if (d->d > 256) {
      return LONGATTN_ERR_UNSUPPORTED;
    }
  }

  a.B = d->batch;
  a.H = d->heads;
  a.n = d->n;
  a.g = d->n_global;
  a.band_on = band_off ? 0 : 1;
  a.wl = band_off ? 0 : std::min(d->win_left, d->n);  // extents beyond n reach no further key
  a.wr = band_off ? 0 : std::min(d->win_right, d->n);
  a.block = has_layout ? d->block : 0;
  a.max_kb = has_layout ? d->max_kb : 0;
  a.scale = d->scale;
  a.scale_log2 = d->scale * 1.44269504088896340736f;

  // Dilation: one value for all heads, or a per-head table carried in the kernel arguments.
  // Without a window the dilation changes nothing, so it is dropped.
  bool uniform = true;
  int dil0 = 1;
  if (d->dilation && a.band_on && d->heads > 0) {
    dil0 = d->dilation[0];
    for (int h = 1; h < d->heads; ++h) uniform = uniform && d->dilation[h] == dil0;
  }
  if (!uniform) {
    if (d->heads > kMaxTableHeads) return LONGATTN_ERR_UNSUPPORTED;
    for (int h = 0; h < d->heads; ++h)
      if (d->dilation[h] > 255) return LONGATTN_ERR_UNSUPPORTED;
  }
  a.uniform_dil = uniform ? dil0 : 0;
  if (!uniform)
    for (int h = 0; h < d->heads; ++h) a.dil[h] = (uint8_t)d->dilation[h];

  p.empty = (a.B == 0 || a.H == 0 || a.n == 0);
  if (p.empty) return LONGATTN_OK;

  if (p.bf16 && for_forward) {
    p.mode = has_layout ? kLayout : kBand;
    const int qt = main_rows_per_workgroup(p.mode, d->d, a.block);
    auto tiles_of_head = [&](int dl) -> long {
      if (p.mode == kLayout) return a.n / a.block;
      long t = 0;
      for (int r = 0; r < dl && r < a.n; ++r) {
        const long n_r = (a.n - r + dl - 1) / dl;
        t += (n_r + qt - 1) / qt;
      }
      return t;
    };
    long per_b = 0;
    if (uniform) {
      const long th = tiles_of_head(dil0);
      a.tile_off[0] = 0;
      a.tile_off[1] = (int)th;
      per_b = th * a.H;
      a.head_tiles = (int)th;
    } else {
      // heads of different dilations often still take the same number of workgroups (n a
      // multiple of dilation x rows per workgroup); the kernels then divide instead of searching
      const long th0 = tiles_of_head(a.dil[0]);
      bool same = true;
      a.tile_off[0] = 0;
      for (int h = 0; h < a.H; ++h) {
        const long th = tiles_of_head(a.dil[h]);
        same = same && th == th0;
        per_b += th;
        a.tile_off[h + 1] = (int)per_b;
      }
      a.head_tiles = same ? (int)th0 : 0;
    }
    if (per_b * a.B > 0x7fffffffL) return LONGATTN_ERR_UNSUPPORTED;
    a.tiles_per_b = (int)per_b;
    p.grid_main = per_b * a.B;
    if (a.g > 0) {
      // global rows: the same launch adds workgroups of qt global rows x chunk_keys keys
      a.chunk_keys = chunk_keys;
      a.chunks = (a.n + chunk_keys - 1) / chunk_keys;
      const long grid_g = (long)a.B * a.H * ((a.g + qt - 1) / qt) * a.chunks;
      if (grid_g + p.grid_main > 0x7fffffffL || (long)a.B * a.H * a.g > 0x7fffffffL)
        return LONGATTN_ERR_UNSUPPORTED;
      a.grid_rows = (int)grid_g;
      // global-row workgroups may follow the XCDs' main work when it splits evenly over them
      a.rows_by_xcd =
          (a.head_tiles > 0 && ((long)a.B * a.H) % 8 == 0 && p.grid_main % 8 == 0) ? 1 : 0;
      // partial outputs, then their (m, l) pairs
      p.part_floats = (size_t)a.B * a.H * a.g * a.chunks * (size_t)(d->d + 2);
      p.ws_bytes = p.part_floats * sizeof(float);
    }
  } else if (for_forward) {
    if ((long)a.B * a.H * a.n / 4 + 1 > 0x7fffffffL) return LONGATTN_ERR_UNSUPPORTED;
  }
  return LONGATTN_OK;
}

// LONGATTN_DEBUG=1: check the device-side index contents on the host before launching.
longattn_status debug_check(const longattn_desc* d, hipStream_t s) {
  if (hipStreamSynchronize(s) != hipSuccess) return LONGATTN_ERR_HIP;
  if (d->n_global > 0) {
    std::vector<int32_t> g((size_t)d->batch * d->n_global);
    if (hipMemcpy(g.data(), d->global_idx, g.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return LONGATTN_ERR_HIP;
    for (int b = 0; b < d->batch; ++b)
      for (int c = 0; c < d->n_global; ++c) {
        const int32_t x = g[(size_t)b * d->n_global + c];
        if (x < 0 || x >= d->n) return LONGATTN_ERR_INVALID_ARG;
        if (c > 0 && x <= g[(size_t)b * d->n_global + c - 1]) return LONGATTN_ERR_INVALID_ARG;
      }
  }
  if (d->block_layout && d->max_kb > 0) {
    const int nb = d->n / d->block;
    std::vector<int32_t> l((size_t)d->heads * nb * d->max_kb);
    if (hipMemcpy(l.data(), d->block_layout, l.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return LONGATTN_ERR_HIP;
    for (size_t r = 0; r < l.size() / d->max_kb; ++r) {
      std::vector<int32_t> row(l.begin() + r * d->max_kb, l.begin() + (r + 1) * d->max_kb);
      for (int32_t x : row)
        if (x < -1 || x >= nb) return LONGATTN_ERR_INVALID_ARG;
      std::sort(row.begin(), row.end());
      for (size_t e = 1; e < row.size(); ++e)
        if (row[e] >= 0 && row[e] == row[e - 1]) return LONGATTN_ERR_INVALID_ARG;
    }
  }
  return LONGATTN_OK;
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

}  // namespace

// ------------------------------------------------------------------------------ backward
namespace {

// The backward pass.  bf16 with d in {64, 128} (window or layout, within the forward's bf16
// limits and at most 1024 layout blocks) runs on the matrix-core kernels (same work decomposition as the forward: prep, dQ kernel, dK/dV kernel, global-row
// combines); everything else on the per-row kernels (Drow, then dQ per query row and dK, dV per
// key column).  Workspace: matrix-core path: Drow and lse2 per row (each padded to 4 floats) and
// fp32 partials of the global rows (dQ: B*H*g*chunks*d; dK, dV: twice that); per-row path: Drow.
struct BwdPlan {
  Plan p;
  bool mfma = false;
  size_t rows_pad = 0;  // floats per per-row array (matrix-core path)
};

longattn_status plan_backward(const longattn_desc* d, BwdPlan* B) {
  Plan& p = B->p;
  bool fast = d && d->dtype == LONGATTN_BF16 && (d->d == 64 || d->d == 128) &&
              (!d->block_layout || (d->block > 0 && d->n / d->block <= kBwdMaxLayoutBlocks));
  longattn_status st = LONGATTN_OK;
  if (fast) {
    st = plan_call(d, true, &p);
    if (st == LONGATTN_ERR_UNSUPPORTED) fast = false;  // limits of the matrix-core kernels
    else if (st != LONGATTN_OK) return st;
  }
  if (!fast) {
    st = plan_call(d, false, &p);
    if (st != LONGATTN_OK) return st;
    if (d->d > 256) return LONGATTN_ERR_UNSUPPORTED;
    if ((long)p.a.B * p.a.H * p.a.n / 4 + 1 > 0x7fffffffL) return LONGATTN_ERR_UNSUPPORTED;
  }
  B->mfma = fast;
  const size_t rows = (size_t)p.a.B * p.a.H * p.a.n;
  if (p.empty) {
    p.ws_bytes = 0;
  } else if (fast) {
    B->rows_pad = (rows + 3) & ~(size_t)3;
    const size_t part = (size_t)p.a.B * p.a.H * p.a.g * p.a.chunks * (size_t)d->d;
    p.ws_bytes = (2 * B->rows_pad + 3 * part) * sizeof(float);
  } else {
    p.ws_bytes = rows * sizeof(float);
  }
  return LONGATTN_OK;
}

}  // namespace

// ------------------------------------------------------------------------------ TGlobal
namespace {

struct TgPlan {
  TgArgs a;
  size_t y_floats = 0;     // side pass: normalised aggregates [B][G][d_model] (bf16; counted
                           // here in floats, so half of it is slack)
  size_t bias_floats = 0;  // attention: per-head bias vectors
  size_t ws_bytes = 0;
  bool empty = false;
};

longattn_status plan_tglobal(const longattn_tglobal_desc* d, TgPlan* P) {
  if (!d) return LONGATTN_ERR_INVALID_ARG;
  if (d->batch < 0 || d->heads < 1 || d->n < 0 || d->d < 1 || d->d_model < 1)
    return LONGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(d->scale) || !(d->scale > 0.f)) return LONGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(d->eps) || d->eps < 0.f) return LONGATTN_ERR_INVALID_ARG;
  if (d->radius < 0 || d->block < 1 || d->num_buckets < 4 || d->num_buckets % 2 != 0 ||
      d->max_distance < 1)
    return LONGATTN_ERR_INVALID_ARG;
  if (d->d != 64 && d->d != 128) return LONGATTN_ERR_UNSUPPORTED;
  if (d->radius > kTgMaxRadius || d->max_distance > kTgMaxMd || d->num_buckets > 256 ||
      d->d_model > kTgMaxDm || d->d_model % 64 != 0)
    return LONGATTN_ERR_UNSUPPORTED;
  if ((long)d->n * d->d * 2 > 0x7fffffffL || (long)d->heads * d->d > 0x7fffffffL / 2)
    return LONGATTN_ERR_UNSUPPORTED;
  const long tiles = ((long)d->n + 127) / 128;
  if ((long)d->batch * d->heads * tiles > 0x7fffffffL) return LONGATTN_ERR_UNSUPPORTED;
  // the projections address W [d_model][heads*d] with 32-bit byte offsets and count the global
  // tokens of all samples in int32
  if ((long)d->d_model * d->heads * d->d * 2 > 0x7fffffffL ||
      (long)d->batch * std::max(1, d->n / d->block) > 0x7fffffffL - 64)
    return LONGATTN_ERR_UNSUPPORTED;
  TgPlan& p = *P;
  p = TgPlan();
  TgArgs& a = p.a;
  std::memset(&a, 0, sizeof(a));
  a.B = d->batch;
  a.H = d->heads;
  a.n = d->n;
  a.D = d->d;
  a.dm = d->d_model;
  a.blk = d->block;
  a.G = std::max(1, d->n / d->block);
  a.radius = std::min(d->radius, std::max(d->n - 1, 0));
  a.rl = a.radius + 191;
  a.md = d->max_distance;
  a.nb = d->num_buckets;
  a.scale_log2 = d->scale * 1.44269504088896340736f;
  a.eps = d->eps;
  a.kpad = d->key_pad;
  p.empty = a.B == 0 || a.n == 0;
  p.y_floats = (size_t)a.B * a.G * a.dm;
  p.bias_floats = (size_t)a.H * (2 * a.rl + 1 + 2 * a.md + 1);
  p.ws_bytes = p.empty ? 0 : std::max(p.y_floats, p.bias_floats) * sizeof(float);
  return LONGATTN_OK;
}

}  // namespace

// ------------------------------------------------------------------------------ decode
namespace {

struct DecodePlan {
  DecodeArgs a;
  size_t ws_bytes = 0;
  bool empty = false;
};

longattn_status plan_decode(const longattn_decode_desc* d, DecodePlan* P) {
  if (!d) return LONGATTN_ERR_INVALID_ARG;
  if (d->batch < 0 || d->heads < 0 || d->d < 1) return LONGATTN_ERR_INVALID_ARG;
  if (d->dtype != LONGATTN_BF16 && d->dtype != LONGATTN_F32) return LONGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(d->scale) || !(d->scale > 0.f)) return LONGATTN_ERR_INVALID_ARG;
  if (d->window < 1 || d->n_queries < 1 || d->cache_len < 1) return LONGATTN_ERR_INVALID_ARG;
  if (d->ring != 0 && d->ring != 1) return LONGATTN_ERR_INVALID_ARG;
  // a rolling buffer must hold every position the rows can reach
  if (d->ring && (long)d->window + d->n_queries - 1 > d->cache_len) return LONGATTN_ERR_INVALID_ARG;
  if (d->batch > 0 && d->heads > 0 && !d->positions) return LONGATTN_ERR_INVALID_ARG;
  if (d->d % 8 != 0 || d->d > kDecodeMaxDim || d->n_queries > kDecodeMaxQueries)
    return LONGATTN_ERR_UNSUPPORTED;
  const long elem = d->dtype == LONGATTN_BF16 ? 2 : 4;
  if ((long)d->cache_len * d->d * elem > 0x7fffffffL) return LONGATTN_ERR_UNSUPPORTED;
  const long span = (long)d->window + d->n_queries - 1;  // positions of the union of windows
  const long bh = (long)d->batch * d->heads;
  const DecodeConfig cfg = decode_config(d->dtype == LONGATTN_BF16, d->d, span, bh);
  const long chunks = cfg.chunks;
  const long rows = bh * d->n_queries;
  if ((long)d->batch * d->heads * chunks > 0x7fffffffL || chunks > 0x7fffffffL)
    return LONGATTN_ERR_UNSUPPORTED;
  DecodePlan& p = *P;
  p = DecodePlan();
  DecodeArgs& a = p.a;
  std::memset(&a, 0, sizeof(a));
  a.B = d->batch;
  a.H = d->heads;
  a.d = d->d;
  a.m = d->n_queries;
  a.window = d->window;
  a.cache_len = d->cache_len;
  a.ring = d->ring;
  a.chunks = (int)chunks;
  a.waves = cfg.waves;
  a.scale_log2 = d->scale * 1.44269504088896340736f;
  a.positions = d->positions;
  p.empty = rows == 0;
  p.ws_bytes = (p.empty || !cfg.merge) ? 0
                                        : (size_t)rows * chunks * (size_t)(d->d + 2) * sizeof(float);
  return LONGATTN_OK;
}

}  // namespace

extern "C" {

longattn_status longattn_workspace_size(const longattn_desc* desc, size_t* bytes) {
  if (!bytes) return LONGATTN_ERR_INVALID_ARG;
  Plan p;
  const longattn_status st = plan_call(desc, true, &p, forward_chunk_keys(desc));
  if (st != LONGATTN_OK) return st;
  *bytes = p.ws_bytes;
  return LONGATTN_OK;
}

}  // extern "C"

namespace {

longattn_status forward_impl(const longattn_desc* desc, const void* q, const void* k,
                             const void* v, const void* gate, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* marks, int32_t n_marks, bool debug_allowed = true) {
  if (n_marks != 0 && n_marks != LONGATTN_N_MARKS) return LONGATTN_ERR_INVALID_ARG;
  if (n_marks && !marks) return LONGATTN_ERR_INVALID_ARG;
  Plan p;
  longattn_status st = plan_call(desc, true, &p, forward_chunk_keys(desc));
  if (st != LONGATTN_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto ev = [&](int i) -> hipEvent_t {
    return n_marks ? reinterpret_cast<hipEvent_t>(marks[i]) : nullptr;
  };
  auto mark = [&](int i) -> bool { return !n_marks || hipEventRecord(ev(i), s) == hipSuccess; };
  if (p.empty) {
    for (int i = 0; i < n_marks; ++i)
      if (!mark(i)) return LONGATTN_ERR_HIP;
    return LONGATTN_OK;
  }
  if (!q || !k || !v || !out) return LONGATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return LONGATTN_ERR_ALIGNMENT;
  if (gate && !aligned16(gate)) return LONGATTN_ERR_ALIGNMENT;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return LONGATTN_ERR_WORKSPACE;
  if (debug_allowed && debug_enabled()) {
    st = debug_check(desc, s);
    if (st != LONGATTN_OK) return st;
  }

  FwdArgs& a = p.a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.gidx = desc->n_global > 0 ? desc->global_idx : nullptr;
  a.kpad = desc->key_pad;
  a.layout = desc->block_layout;
  a.part = static_cast<float*>(workspace);
  a.gate = static_cast<const uint16_t*>(gate);

  // bf16: one launch computes every non-global row and, in extra workgroups, the global rows'
  // per-chunk partials; the combine then writes the global rows (overwriting what the main work
  // produced for them).  Marks are attached to the kernels' own dispatches, so they time the
  // kernels themselves.
  hipError_t e = hipSuccess;
  if (p.bf16) {
    e = launch_attention(a, desc->d, p.mode, p.grid_main + a.grid_rows, s, {ev(0), ev(1)});
    if (e != hipSuccess) return LONGATTN_ERR_HIP;
    if (a.g > 0) {
      e = launch_global_combine(a, desc->d, s, {ev(2), ev(3)});
      if (e != hipSuccess) return LONGATTN_ERR_HIP;
    } else if (!mark(2) || !mark(3)) {
      return LONGATTN_ERR_HIP;
    }
  } else {
    if (!mark(0)) return LONGATTN_ERR_HIP;
    e = launch_rowwise_f32(a, desc->d, s);
    if (e != hipSuccess || !mark(1) || !mark(2) || !mark(3)) return LONGATTN_ERR_HIP;
  }
  return LONGATTN_OK;
}

}  // namespace

extern "C" {

longattn_status longattn_forward_marked(const longattn_desc* desc, const void* q, const void* k,
                                        const void* v, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream,
                                        void* const* marks, int32_t n_marks) {
  return forward_impl(desc, q, k, v, nullptr, out, lse, workspace, workspace_bytes, stream,
                      marks, n_marks);
}

longattn_status longattn_forward(const longattn_desc* desc, const void* q, const void* k,
                                 const void* v, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return forward_impl(desc, q, k, v, nullptr, out, lse, workspace, workspace_bytes, stream,
                      nullptr, 0);
}

longattn_status longattn_forward_gated(const longattn_desc* desc, const void* q, const void* k,
                                       const void* v, const void* gate, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate) return LONGATTN_ERR_INVALID_ARG;
  return forward_impl(desc, q, k, v, gate, out, lse, workspace, workspace_bytes, stream,
                      nullptr, 0);
}

}  // extern "C"

// ------------------------------------------------------------------------------ no allocation
// Scratch of longattn_forward_noalloc: the global-row partials of a forward pass, in a device
// array of the library's own.  Each GPU the library runs on holds one copy of it until the
// process ends.  Host code must not take the array's address directly (on the host, its name
// stands for a host-side shadow): each device's address comes from hipGetSymbolAddress, resolved
// once per device with that device current and kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[LONGATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device that owns `stream` (the current device for the
// null stream).
longattn_status scratch_for(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return LONGATTN_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return LONGATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return LONGATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return LONGATTN_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return LONGATTN_ERR_HIP;
    if (e != hipSuccess || !ptr) return LONGATTN_ERR_HIP;
    scratch_addr[dev] = ptr;
  }
  *out = scratch_addr[dev];
  return LONGATTN_OK;
}

}  // namespace

extern "C" {

longattn_status longattn_forward_noalloc(const longattn_desc* desc, const void* q, const void* k,
                                         const void* v, void* out, float* lse, void* stream) {
  Plan p;
  longattn_status st = plan_call(desc, true, &p, forward_chunk_keys(desc));
  if (st != LONGATTN_OK) return st;
  if (p.ws_bytes > (size_t)LONGATTN_NOALLOC_SCRATCH_BYTES) return LONGATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p.ws_bytes > 0 && !p.empty) {
    st = scratch_for(reinterpret_cast<hipStream_t>(stream), &ws);
    if (st != LONGATTN_OK) return st;
  }
  // every partial the combine reads is written by the same pass first: nothing to clear
  return forward_impl(desc, q, k, v, nullptr, out, lse, ws, p.ws_bytes, stream, nullptr, 0,
                      /*debug_allowed=*/false);
}

longattn_status longattn_count_entries(const longattn_desc* desc, int64_t* entries_out,
                                       void* stream) {
  if (!entries_out) return LONGATTN_ERR_INVALID_ARG;
  Plan p;
  const longattn_status st = plan_call(desc, false, &p);
  if (st != LONGATTN_OK) return st;
  FwdArgs& a = p.a;
  a.gidx = desc->n_global > 0 ? desc->global_idx : nullptr;
  a.kpad = desc->key_pad;
  a.layout = desc->block_layout;
  if (p.empty) {
    a.B = a.H = a.n = 0;
  }
  const hipError_t e = launch_count_entries(a, entries_out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LONGATTN_OK : LONGATTN_ERR_HIP;
}


longattn_status longattn_backward_workspace_size(const longattn_desc* desc, size_t* bytes) {
  if (!bytes) return LONGATTN_ERR_INVALID_ARG;
  BwdPlan bp;
  const longattn_status st = plan_backward(desc, &bp);
  if (st != LONGATTN_OK) return st;
  *bytes = bp.p.ws_bytes;
  return LONGATTN_OK;
}

longattn_status longattn_backward_marked(const longattn_desc* desc, const void* q,
                                         const void* k, const void* v, const void* out,
                                         const float* lse, const void* dout, void* dq, void* dk,
                                         void* dv, void* workspace, size_t workspace_bytes,
                                         void* stream, void* const* marks, int32_t n_marks) {
  if (n_marks != 0 && n_marks != LONGATTN_BWD_N_MARKS) return LONGATTN_ERR_INVALID_ARG;
  if (n_marks && !marks) return LONGATTN_ERR_INVALID_ARG;
  BwdPlan bp;
  longattn_status st = plan_backward(desc, &bp);
  if (st != LONGATTN_OK) return st;
  Plan& p = bp.p;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto ev = [&](int i) -> hipEvent_t {
    return n_marks ? reinterpret_cast<hipEvent_t>(marks[i]) : nullptr;
  };
  auto mark_all = [&]() -> bool {
    for (int i = 0; i < n_marks; ++i)
      if (hipEventRecord(ev(i), s) != hipSuccess) return false;
    return true;
  };
  if (p.empty) return mark_all() ? LONGATTN_OK : LONGATTN_ERR_HIP;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)
    return LONGATTN_ERR_INVALID_ARG;
  for (const void* x : {q, k, v, out, dout, static_cast<const void*>(dq),
                        static_cast<const void*>(dk), static_cast<const void*>(dv)})
    if (!aligned16(x)) return LONGATTN_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return LONGATTN_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < p.ws_bytes) return LONGATTN_ERR_WORKSPACE;
  if (debug_enabled()) {
    st = debug_check(desc, s);
    if (st != LONGATTN_OK) return st;
  }
  FwdArgs& a = p.a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.lse = const_cast<float*>(lse);  // read only by the backward kernels
  a.gidx = desc->n_global > 0 ? desc->global_idx : nullptr;
  a.kpad = desc->key_pad;
  a.layout = desc->block_layout;
  BwdArgs g;
  g.out = out;
  g.dout = dout;
  g.dq = dq;
  g.dk = dk;
  g.dv = dv;
  g.drow = static_cast<float*>(workspace);
  g.lse2 = nullptr;
  const long rows = (long)a.B * a.H * a.n;
  hipError_t e = hipSuccess;
  if (bp.mfma) {
    g.lse2 = g.drow + bp.rows_pad;
    a.part = g.drow + 2 * bp.rows_pad;
    LaunchEvents le[3];
    for (int i = 0; i < 3 && n_marks; ++i) le[i] = {ev(2 * i), ev(2 * i + 1)};
    e = launch_bwd_mfma(a, g, desc->d, p.mode, p.grid_main + a.grid_rows, s,
                        n_marks ? le : nullptr);
  } else {
    if (n_marks && hipEventRecord(ev(0), s) != hipSuccess) return LONGATTN_ERR_HIP;
    e = launch_bwd_rowdot(g, rows, desc->d, p.bf16, s);
    if (e == hipSuccess && n_marks && hipEventRecord(ev(1), s) != hipSuccess) return LONGATTN_ERR_HIP;
    if (e == hipSuccess && n_marks && hipEventRecord(ev(2), s) != hipSuccess) return LONGATTN_ERR_HIP;
    if (e == hipSuccess) e = launch_bwd_rowwise(a, g, desc->d, p.bf16, s);
    for (int i = 3; i < n_marks && e == hipSuccess; ++i)
      if (hipEventRecord(ev(i), s) != hipSuccess) return LONGATTN_ERR_HIP;
  }
  return e == hipSuccess ? LONGATTN_OK : LONGATTN_ERR_HIP;
}

longattn_status longattn_backward(const longattn_desc* desc, const void* q, const void* k,
                                  const void* v, const void* out, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return longattn_backward_marked(desc, q, k, v, out, lse, dout, dq, dk, dv, workspace,
                                  workspace_bytes, stream, nullptr, 0);
}

longattn_status longattn_gate_lowrank(const longattn_gate_desc* desc, void* out,
                                      const void* w_down, const void* w_up, void* stream) {
  if (!desc) return LONGATTN_ERR_INVALID_ARG;
  if (desc->batch < 0 || desc->heads < 1 || desc->n < 0 || desc->d < 1 || desc->rank < 1)
    return LONGATTN_ERR_INVALID_ARG;
  const long hd = (long)desc->heads * desc->d;
  if (desc->d % 16 != 0 || hd % 32 != 0 || hd > 16384) return LONGATTN_ERR_UNSUPPORTED;
  if (desc->rank != 32 && desc->rank != 64 && desc->rank != 128 && desc->rank != 256)
    return LONGATTN_ERR_UNSUPPORTED;
  const long tokens = (long)desc->batch * desc->n;
  if (tokens * hd > (1L << 46) || (tokens + 127) / 128 > 0x7fffffffL)
    return LONGATTN_ERR_UNSUPPORTED;
  if (tokens == 0) return LONGATTN_OK;
  if (!out || !w_down || !w_up) return LONGATTN_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(w_down) || !aligned16(w_up)) return LONGATTN_ERR_ALIGNMENT;
  GateArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.w_down = static_cast<const uint16_t*>(w_down);
  a.w_up = static_cast<const uint16_t*>(w_up);
  a.B = desc->batch;
  a.H = desc->heads;
  a.n = desc->n;
  a.d = desc->d;
  a.r = desc->rank;
  const hipError_t e = launch_gate_lowrank(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LONGATTN_OK : LONGATTN_ERR_HIP;
}

longattn_status longattn_tglobal_workspace_size(const longattn_tglobal_desc* desc, size_t* bytes) {
  if (!bytes) return LONGATTN_ERR_INVALID_ARG;
  TgPlan p;
  const longattn_status st = plan_tglobal(desc, &p);
  if (st != LONGATTN_OK) return st;
  *bytes = p.ws_bytes;
  return LONGATTN_OK;
}

longattn_status longattn_tglobal_side(const longattn_tglobal_desc* desc, const void* x,
                                      const float* gamma, const void* wk, const void* wv,
                                      void* side_k, void* side_v, uint8_t* side_valid,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  TgPlan p;
  const longattn_status st = plan_tglobal(desc, &p);
  if (st != LONGATTN_OK) return st;
  if (p.empty) return LONGATTN_OK;
  if (!x || !gamma || !wk || !wv || !side_k || !side_v || !side_valid)
    return LONGATTN_ERR_INVALID_ARG;
  for (const void* t : {x, wk, wv, static_cast<const void*>(side_k),
                        static_cast<const void*>(side_v)})
    if (!aligned16(t)) return LONGATTN_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(gamma) & 3u) != 0) return LONGATTN_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < p.ws_bytes) return LONGATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LONGATTN_ERR_ALIGNMENT;  // rows of normalised inputs
  TgArgs& a = p.a;
  a.side_valid = side_valid;
  a.sk_out = static_cast<uint16_t*>(side_k);
  a.sv_out = static_cast<uint16_t*>(side_v);
  const hipError_t e = launch_tglobal_side(
      a, static_cast<const uint16_t*>(x), gamma, static_cast<const uint16_t*>(wk),
      static_cast<const uint16_t*>(wv), static_cast<uint16_t*>(workspace),
      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LONGATTN_OK : LONGATTN_ERR_HIP;
}

longattn_status longattn_tglobal_forward(const longattn_tglobal_desc* desc, const void* q,
                                         const void* k, const void* v, const void* side_k,
                                         const void* side_v, const uint8_t* side_valid,
                                         const float* bias_local, const float* bias_side,
                                         void* out, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  TgPlan p;
  const longattn_status st = plan_tglobal(desc, &p);
  if (st != LONGATTN_OK) return st;
  if (p.empty) return LONGATTN_OK;
  if (!q || !k || !v || !side_k || !side_v || !side_valid || !bias_local || !bias_side || !out)
    return LONGATTN_ERR_INVALID_ARG;
  for (const void* t : {q, k, v, side_k, side_v, static_cast<const void*>(out)})
    if (!aligned16(t)) return LONGATTN_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < p.ws_bytes) return LONGATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LONGATTN_ERR_ALIGNMENT;
  TgArgs& a = p.a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sk = static_cast<const uint16_t*>(side_k);
  a.sv = static_cast<const uint16_t*>(side_v);
  a.side_valid = const_cast<uint8_t*>(side_valid);  // read only by the attention kernel
  a.bias = static_cast<float*>(workspace);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const hipError_t e = launch_tglobal_attention(a, bias_local, bias_side,
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LONGATTN_OK : LONGATTN_ERR_HIP;
}

longattn_status longattn_decode_workspace_size(const longattn_decode_desc* desc, size_t* bytes) {
  if (!bytes) return LONGATTN_ERR_INVALID_ARG;
  DecodePlan p;
  const longattn_status st = plan_decode(desc, &p);
  if (st != LONGATTN_OK) return st;
  *bytes = p.ws_bytes;
  return LONGATTN_OK;
}

longattn_status longattn_decode(const longattn_decode_desc* desc, const void* q,
                                const void* k_cache, const void* v_cache, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan p;
  const longattn_status st = plan_decode(desc, &p);
  if (st != LONGATTN_OK) return st;
  if (p.empty) return LONGATTN_OK;
  if (!q || !k_cache || !v_cache || !out) return LONGATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return LONGATTN_ERR_ALIGNMENT;
  if (p.ws_bytes && (!workspace || workspace_bytes < p.ws_bytes)) return LONGATTN_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (debug_enabled()) {
    if (hipStreamSynchronize(s) != hipSuccess) return LONGATTN_ERR_HIP;
    std::vector<int32_t> pos(desc->batch);
    if (hipMemcpy(pos.data(), desc->positions, pos.size() * 4, hipMemcpyDeviceToHost) !=
        hipSuccess)
      return LONGATTN_ERR_HIP;
    for (int32_t t0 : pos) {
      if (t0 < 0) return LONGATTN_ERR_INVALID_ARG;
      if (!desc->ring && (long)t0 + desc->n_queries - 1 >= desc->cache_len)
        return LONGATTN_ERR_INVALID_ARG;
    }
  }
  DecodeArgs& a = p.a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.lse = lse;
  a.part = static_cast<float*>(workspace);
  const hipError_t e = launch_decode(a, desc->dtype == LONGATTN_BF16, s);
  return e == hipSuccess ? LONGATTN_OK : LONGATTN_ERR_HIP;
}

const char* longattn_status_string(longattn_status status) {
  switch (status) {
    case LONGATTN_OK: return "ok";
    case LONGATTN_ERR_INVALID_ARG: return "invalid argument";
    case LONGATTN_ERR_UNSUPPORTED: return "unsupported by the GPU kernels";
    case LONGATTN_ERR_ALIGNMENT: return "q, k, v or out not 16-byte aligned";
    case LONGATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case LONGATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
