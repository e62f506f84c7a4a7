// C ABI of the fused attention forward library (declared in include/fa.h).
//
// This file holds the host side only: argument checks, the choice of kernel
// variant (rows per wave, waves per workgroup, key tile, key split), the
// per-device workspace registry, and the launch.  It never touches device
// memory: seqused_k is read only by the kernels.  Checks run before any HIP
// call, so every error path works without a GPU (the failure convention of
// the pages: explicit errors, never an implicit fallback --
// "pi05_thor_decoder_fp4_e2e.md", section "Implemented Path"; fail before
// capture, naming the cause -- "GROOT N1.7 update", section "Shared-code
// changes").

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

static_assert(fa::kStaticScratchBytes == FA_STATIC_SCRATCH_BYTES, "one size for the static split scratch");

namespace {

constexpr int kMaxDevices = 64;
constexpr long long kTargetWorkgroups = 256;  // one per compute unit on MI355X
// Key buffers up to this length take split ranges from the grid size alone,
// so a padded buffer and its valid keys split identically (bit-identical
// results); longer buffers size their ranges from the buffer length.
constexpr int kLongKeys = 2048;

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
Workspace g_ws[kMaxDevices];
std::mutex g_ws_mu;

bool supported_d(int D) { return D == 64 || D == 72 || D == 256; }

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// Element strides (batch, sequence, head) of one (B, S, H, D) view.
struct View {
  long long sb, ss, sh;
};
View contiguous(int S, int H, int D) { return View{(long long)S * H * D, (long long)H * D, (long long)D}; }

struct Plan {
  fa::LaunchPlan launch{};
  int Mp = 0;
  int kps = 0;
  int nrb = 0;
  int zmax = 0;
  size_t ws_o_bytes = 0, ws_ml_bytes = 0, ws_bytes = 0;
};

// Packed rows one workgroup covers: nw / kw waves on different rows, each
// row set shared by kw waves that split the keys (kw == 1: every wave has
// its own rows; kw == nw: all waves on the same 16*qt rows).
int rows_per_block(const fa::LaunchPlan& l) { return (l.nw / l.kw) * 16 * l.qt; }

// Fills in the derived fields (row blocks, split count, workspace layout) of
// a plan whose variant and keys-per-split are set.  kps == 0: no split.
void finish_plan(Plan& pl, int B, int Sq, int Sk, int Hq, int Hkv, int causal) {
  const int g = Hq / Hkv;
  pl.Mp = Sq * g;
  const int rows = rows_per_block(pl.launch);
  pl.nrb = (int)cdiv(pl.Mp, rows);
  pl.launch.causal = causal != 0;
  pl.launch.split = pl.kps > 0;
  pl.launch.nsplit = 0;
  pl.zmax = 0;
  pl.ws_o_bytes = pl.ws_ml_bytes = pl.ws_bytes = 0;
  if (!pl.launch.split) return;
  if (causal) {
    // keys of the last row block (the last query attends the whole buffer)
    const long long last = (std::min((long long)pl.nrb * rows, (long long)pl.Mp) - 1) / g + (Sk - Sq) + 1;
    const long long kmax_last = std::max(0ll, std::min((long long)Sk, last));
    pl.zmax = (int)std::max(1ll, cdiv(kmax_last, pl.kps));
  } else {
    pl.launch.nsplit = (int)cdiv(Sk, pl.kps);
    pl.zmax = pl.launch.nsplit;
  }
  const size_t prow = (size_t)B * Hkv * pl.nrb * pl.zmax * rows;
  // Layout: the partial O rows, then the (m, l) pairs.
  pl.ws_o_bytes = (prow * pl.launch.D * sizeof(float) + 255) / 256 * 256;
  pl.ws_ml_bytes = (prow * 2 * sizeof(float) + 255) / 256 * 256;
  pl.ws_bytes = pl.ws_o_bytes + pl.ws_ml_bytes;
}

// Default variant for a shape: a function of the shape only (never of the
// seqused_k values), so equal shapes always run the same kernel.
//  * Head dim 256: key-split workgroups (32 rows, four waves over the keys),
//    which read half the LDS bytes per MFMA of the row-split kernel; 16 rows
//    when the keys are split as well (below).
//  * Smaller head dims: row-split workgroups, one wave per 16 packed rows.
// When the single-pass grid is at most half the compute units, the key
// range is split into fixed-size ranges, merged afterwards by the
// combine kernel.  The range size depends on the grid size only, not on the
// key buffer length, so a padded buffer and the same keys without the
// padding are split at the same boundaries (the extra ranges of the padded
// one are empty and skipped by the merge): their results are bit-identical.
Plan default_plan(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal) {
  Plan pl;
  pl.launch.D = D;
  const long long BH = (long long)B * Hkv;
  const long long Mp = (long long)Sq * (Hq / Hkv);
  if (D == 256) {
    pl.launch.qt = 2;
    pl.launch.nw = 4;
    pl.launch.kw = 4;
    pl.launch.bn = 32;
    pl.launch.nst = 2;  // piecewise refill (measured against whole-tile buffers: causal 2048 prefill 32.9 -> 30.7 us)
  } else {
    pl.launch.qt = 1;
    pl.launch.nw = 4;
    pl.launch.kw = 1;
    pl.launch.bn = 64;
    pl.launch.nst = 2;
  }
  const int rows = rows_per_block(pl.launch);
  const long long base = cdiv(Mp, rows) * BH;
  // Row-split: 128-key tiles (half the trips, barriers and row reductions
  // per key) when the single-pass grid fits the compute units in one round
  // and the buffer holds at least one such tile.  Their 96 KB of stages allow
  // one workgroup per compute unit, so larger grids keep 64-key tiles, with
  // which two or three workgroups share a compute unit.
  if (D != 256 && base <= kTargetWorkgroups && Sk >= 128) pl.launch.bn = 128;
  pl.kps = 0;
  if (base <= kTargetWorkgroups / 2 && Sk > kLongKeys) {
    // Long key buffers: about 32 ranges per row block (fewer when the grid
    // would exceed one workgroup per compute unit), each a power-of-two
    // number of keys.  Here the loop dominates, so D256 keeps 32-row
    // workgroups (half the K/V traffic per MFMA of 16-row ones) unless the
    // rows fit in 16 or the split grid would still fill under half the
    // compute units (32 packed rows over 4000 keys: 12.5 -> 10.8 us).  Measured against the short-buffer rule below: 131072
    // keys, 128 packed rows 242 -> 82 us; decode over 32768 keys 45.8 ->
    // 19.5 us; 16384 keys, 128 rows 37.7 -> 22.6 us; D64 over 65536 keys
    // 72.8 -> 23.5 us.  Ranges of 256 keys rather than 512 where the buffer
    // allows: D64 decode over 4096 keys 9.2 -> 8.4 us.
    const long long splits = std::min(32ll, std::max(2ll, kTargetWorkgroups / base));
    int kps = 256;
    while ((long long)kps * splits < Sk) kps *= 2;
    pl.kps = kps;
    if (D == 256 && (Mp <= 16 || base * splits < kTargetWorkgroups / 2)) pl.launch.qt = 1;
  } else if (base <= kTargetWorkgroups / 2) {
    if (D == 256) {
      // Grids of at most half the compute units at head dim 256 take 16-row
      // key-split workgroups: twice the workgroups, each with half the rows.
      // Measured against 32-row workgroups: the 41-row action expert shape
      // 12.0 -> 10.0 us, a causal 64-row chunk 12.0 -> 11.0 us, decode 9.5 ->
      // 8.4 us; without a split, 4096 packed rows over 512 keys 11.6 -> 8.8
      // us.  The range size follows the 16-row grid.
      // A 16-row grid of more than half the compute units is not split
      // further (8 x 41 rows over 1056 keys: 24.8 -> 16.5 us).
      const long long base1 = cdiv(Mp, 16) * BH;
      const int kps = base1 <= 4 ? 128 : (base1 <= 64 ? 256 : 512);
      if (Sk > kps && base1 <= kTargetWorkgroups / 2) pl.kps = kps;
      pl.launch.qt = 1;
    } else {
      const int kps = base <= 32 ? 128 : (base <= 64 ? 256 : 512);
      if (Sk > kps) pl.kps = kps;
    }
  }
  if (D == 256 && !causal && pl.kps == 0 && base > 3 * kTargetWorkgroups) {
    // More than three rounds of 32-row key-split blocks: every compute unit
    // would pull the whole K/V of its head from L2 per 32 rows.  Row-split
    // blocks of four 32-row waves share each K/V tile among 128 rows
    // (4 x 1024 x 1024 prefix rows, 8/1 heads: 65.1 -> 46.3 us, the ring
    // scheme 54.0; against the ring: 896 blocks 45.3 -> 41.4 us, 960 blocks
    // 49.9 -> 43.9 and 47.9 -> 46.2, 1000 blocks 52.9 -> 46.4).
    pl.launch.qt = 2;
    pl.launch.nw = 4;
    pl.launch.kw = 1;
    pl.launch.bn = 32;
    pl.launch.nst = 2;
  } else if (D == 256 && !causal && pl.kps == 0 && base > kTargetWorkgroups) {
    // Up to three rounds: the key-split kernel's ring buffer scheme, two
    // workgroups per compute unit (the 128-row row-split blocks above take
    // 45.9 us at 768 blocks against the ring's 41.7, 40.7 against 34.5 at
    // 660).  Measured against row-split blocks of
    // four 16-row waves over 64-key tiles and against the two-buffer
    // key-split kernel (us per call): 2 x 768 x 768 prefix rows 25.2 / 21.5
    // -> 19.7; 2 x 1024 x 1024 32.3 / 27.2 -> 27.0; 3 x 1024 x 1024 62.9 /
    // 45.1 -> 41.9; 3 x 700 x 700 45.5 / 30.3 -> 27.9; 1536 x 1536 44.8 /
    // 34.5 -> 32.6; 1024 x 1024 with 16/2 heads 32.8 / 27.3 -> 27.2.
    pl.launch.nst = 3;
  }
  if (D == 256 && causal && pl.kps == 0 && pl.launch.kw == 4 && BH == 1 &&
      base > 2 * kTargetWorkgroups - kTargetWorkgroups / 8 && base <= 2 * kTargetWorkgroups) {
    // Causal grids of one (batch, kv head) with about two row blocks per
    // compute unit: the ring buffer scheme (80 KiB of LDS, two waves per
    // SIMD) with a heavy and a light row block on each compute unit, so
    // that one workgroup's prologue and merge overlap the other's tiles
    // (causal 2048 prefill 28.4 -> 27.2 us).  With fewer blocks the
    // heaviest ones run alone on their compute units, where the ring's
    // half-size buffers are slower (384 blocks: 19.7 -> 21.9 us).
    pl.launch.nst = 3;
  }
  if (D != 256 && pl.kps == 0) {
    // Single-pass row-split grids: two key groups of waves on the same rows
    // (each taking every other 64-key tile, merged in LDS) once a row sees
    // enough keys, so that two waves share each SIMD.  Long key ranges keep
    // 64-row blocks (four row waves); grids of at most half the compute
    // units take 32-row blocks (two row waves), twice the workgroups.
    // Measured against one group: 16 heads of 1024 x 1024 at D72 13.7 ->
    // 12.3 us, 768 x 768 at D72 11.0 -> 10.0 us, causal 1024 x 1024 at D72
    // 14.7 -> 12.8 us, causal 8 heads of 2048 at D64 20.1 -> 17.7 us, one
    // 256-token view of 16 heads at D72 5.44 -> 4.96 us.
    const long long keys = causal ? Sk / 2 : Sk;  // keys per row on average
    if (base <= kTargetWorkgroups && Sk >= 768) {
      pl.launch.nw = 8;
      pl.launch.kw = 2;
      pl.launch.bn = 64;
    } else if (base <= kTargetWorkgroups / 2 && keys >= 256) {
      pl.launch.nw = 4;
      pl.launch.kw = 2;
      pl.launch.bn = 64;
    } else if (!causal && base >= 4 * kTargetWorkgroups && Sk >= 1024) {
      // Four or more rounds of 64-row blocks over long key ranges: 32 rows
      // per wave (128-row blocks) halve the LDS reads per row.  Measured
      // against 16 rows per wave: 1024 blocks of 2048 x 2048 at D72 93 ->
      // 56 us (128-key tiles) and 32/8 GQA heads at D64 53.4 -> 45.4 us;
      // 2048 blocks of 1024 keys at D64 56.7 -> 46.6 us.  At 512 blocks and
      // for causal grids one 16-row wave per SIMD stays ahead.
      pl.launch.qt = 2;
    } else if (D == 64 && base > kTargetWorkgroups && base < 4 * kTargetWorkgroups && Sk >= 1024) {
      // Two or three rounds at D64 over long key ranges: 128-key tiles (two
      // rounds of 1024 x 1024, 16 heads: 18.2 -> 15.3 us; causal 4096 x
      // 4096, 8 heads: 53.2 -> 48.7 us).  At D72 the larger stages cost more
      // than they save (4 x 1024 x 1024, 8 heads: 20.6 -> 27.2 us).
      pl.launch.bn = 128;
    }
  }
  finish_plan(pl, B, Sq, Sk, Hq, Hkv, causal);
  return pl;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

int check_shape(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal) {
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || D < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  const long long qn = (long long)B * Sq * Hq * D;
  const long long kn = (long long)B * Sk * Hkv * D;
  const long long pn = (long long)Sq * (Hq / Hkv);
  if (qn > INT32_MAX || kn > INT32_MAX || pn > INT32_MAX / 2) return FA_ERR_SHAPE;
  if ((long long)B * Hkv > 65535) return FA_ERR_SHAPE;  // grid.y limit
  if ((long long)Sk * Hkv * D * 2 >= (1ll << 31)) return FA_ERR_SHAPE;  // K/V bytes per batch entry (32-bit offsets)
  if (!supported_d(D)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_args(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk,
               int Hq, int Hkv, int D, int causal, const int32_t* seqused_k, float scale) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return FA_ERR_NULL;
  int rc = check_shape(B, Sq, Sk, Hq, Hkv, D, causal);
  if (rc != FA_OK) return rc;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_ALIGN;
  if ((lse != nullptr && !aligned(lse, 4)) || (seqused_k != nullptr && !aligned(seqused_k, 4)))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)B * Sq * Hq * D * 2, kb = (size_t)B * Sk * Hkv * D * 2;
  if (overlap(out, qb, q, qb) || overlap(out, qb, k, kb) || overlap(out, qb, v, kb)) return FA_ERR_ALIAS;
  // seqused_k is read by workgroups that may start after others have
  // written their output rows, so it may not share a byte with out or lse.
  const size_t sb = (size_t)B * sizeof(int32_t);
  if (seqused_k != nullptr && overlap(out, qb, seqused_k, sb)) return FA_ERR_ALIAS;
  if (lse != nullptr) {
    const size_t lb = (size_t)B * Hq * Sq * sizeof(float);
    if (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
        overlap(lse, lb, out, qb) || (seqused_k != nullptr && overlap(lse, lb, seqused_k, sb)))
      return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// Byte range [lo, hi) touched by a (B, S, H, D) view of 16-bit elements.
void view_span(const void* base, int B, int S, int H, int D, const View& w, uintptr_t& lo, uintptr_t& hi) {
  lo = (uintptr_t)base;
  hi = lo + 2 * (uintptr_t)((B - 1) * w.sb + (S - 1) * w.ss + (H - 1) * w.sh + D);
}

bool spans_overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

// Every (batch, position, head) row of the view is disjoint from the others:
// ordered by stride, each dimension of extent > 1 steps past everything the
// smaller ones span.
bool rows_disjoint(int B, int S, int H, int D, const View& w) {
  struct Dim {
    long long stride, extent;
  } d[3] = {{w.sb, B}, {w.ss, S}, {w.sh, H}};
  std::sort(d, d + 3, [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
  long long span = D;  // elements covered by the inner dimensions
  for (const Dim& x : d) {
    if (x.extent == 1) continue;
    if (x.stride < span) return false;
    span = x.stride * (x.extent - 1) + span;
  }
  return true;
}

// Checks of fa_fwd_strided (the strided form of check_args).
int check_strided(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk,
                  int Hq, int Hkv, int D, const View& vq, const View& vk, const View& vv, const View& vo,
                  int dtype, int causal, const int32_t* seqused_k, float scale) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return FA_ERR_NULL;
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if ((long long)B * Hkv > 65535 || (long long)Sq * (Hq / Hkv) > INT32_MAX / 2) return FA_ERR_SHAPE;
  const View* views[4] = {&vq, &vk, &vv, &vo};
  for (const View* w : views)
    if (w->sb < 0 || w->ss < 0 || w->sh < 0 || w->ss >= (1ll << 31) || w->sh >= (1ll << 31)) return FA_ERR_SHAPE;
  // 32-bit offsets inside the kernels: keys of one (batch, kv head) and the
  // query rows of one batch entry.
  if ((long long)Sk * vk.ss * 2 >= (1ll << 31) || (long long)Sk * vv.ss * 2 >= (1ll << 31)) return FA_ERR_SHAPE;
  if (((long long)(Sq - 1) * vq.ss + (long long)(Hq - 1) * vq.sh + D) * 2 >= (1ll << 31)) return FA_ERR_SHAPE;
  if (!supported_d(D)) return FA_ERR_UNSUPPORTED;
  if (dtype != fa::kBf16 && dtype != fa::kF16) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  // Key rows of one head may not overlap (a row ends before the next starts),
  // and every output row is written once.
  if ((Sk > 1 && (vk.ss < D || vv.ss < D)) || !rows_disjoint(B, Sq, Hq, D, vo)) return FA_ERR_SHAPE;
  // 16-byte rows: 16-byte aligned bases and strides in multiples of 8 elements.
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_ALIGN;
  for (const View* w : views)
    if (w->sb % 8 != 0 || w->ss % 8 != 0 || w->sh % 8 != 0) return FA_ERR_ALIGN;
  if ((lse != nullptr && !aligned(lse, 4)) || (seqused_k != nullptr && !aligned(seqused_k, 4)))
    return FA_ERR_ALIGN;
  uintptr_t q0, q1, k0, k1, v0, v1, o0, o1;
  view_span(q, B, Sq, Hq, D, vq, q0, q1);
  view_span(k, B, Sk, Hkv, D, vk, k0, k1);
  view_span(v, B, Sk, Hkv, D, vv, v0, v1);
  view_span(out, B, Sq, Hq, D, vo, o0, o1);
  if (spans_overlap(o0, o1, q0, q1) || spans_overlap(o0, o1, k0, k1) || spans_overlap(o0, o1, v0, v1))
    return FA_ERR_ALIAS;
  const uintptr_t s0 = (uintptr_t)seqused_k, s1 = s0 + (uintptr_t)B * sizeof(int32_t);
  if (seqused_k != nullptr && spans_overlap(o0, o1, s0, s1)) return FA_ERR_ALIAS;
  if (lse != nullptr) {
    const uintptr_t l0 = (uintptr_t)lse, l1 = l0 + (uintptr_t)B * Hq * Sq * sizeof(float);
    if (spans_overlap(l0, l1, q0, q1) || spans_overlap(l0, l1, k0, k1) || spans_overlap(l0, l1, v0, v1) ||
        spans_overlap(l0, l1, o0, o1) || (seqused_k != nullptr && spans_overlap(l0, l1, s0, s1)))
      return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// Variant given by the caller: checked against the compiled set.
int variant_plan(Plan& pl, int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal, int qt, int nw, int kw,
                 int bn, int nst, int kps) {
  if (!fa::variant_exists(D, qt, nw, kw, bn, nst, fa::kBf16)) return FA_ERR_UNSUPPORTED;
  pl.launch.dtype = fa::kBf16;
  if (kps < 0 || (kps > 0 && kps % bn != 0)) return FA_ERR_UNSUPPORTED;
  pl.launch.D = D;
  pl.launch.qt = qt;
  pl.launch.nw = nw;
  pl.launch.kw = kw;
  pl.launch.bn = bn;
  pl.launch.nst = nst;
  pl.kps = kps;
  finish_plan(pl, B, Sq, Sk, Hq, Hkv, causal);
  return FA_OK;
}

// A packed variable-length batch (fa_fwd_varlen): device offsets and row counts.
struct Packed {
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

// Where the split-KV partials of a call go: the workspace registered for
// the current device, or the library's static scratch (fa_fwd_static).
enum class Scratch { kRegistered, kStatic };

int run(const Plan& pl, const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq,
        int Sk, int Hq, int Hkv, const View& vq, const View& vk, const View& vv, const View& vo,
        const int32_t* seqused_k, float scale, hipStream_t stream, const Packed& packed = Packed(),
        void* fp4_out = nullptr, void* fp4_sf = nullptr, Scratch where = Scratch::kRegistered) {
  fa::FwdParams p{};
  p.fp4_out = static_cast<uint8_t*>(fp4_out);
  p.fp4_sf = static_cast<uint8_t*>(fp4_sf);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.seqused = seqused_k;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.g = Hq / Hkv;
  p.g_m = 0xffffffffu / (uint32_t)p.g;
  p.Mp = pl.Mp;
  p.coff = Sk - Sq;
  p.lse_hs = Sq;
  p.lse_bs = (long long)Hq * Sq;
  if (packed.cu_q != nullptr) {
    p.cu_q = packed.cu_q;
    p.cu_k = packed.cu_k;
    p.total_q = packed.total_q;
    p.total_k = packed.total_k;
    p.lse_hs = packed.total_q;
    p.lse_bs = 0;  // a sequence's rows are located by its query offset
    // Grids are planned for the longest sequences; a sequence may pair any
    // query count with up to Sk keys, so causal blocks plan for all Sk keys.
    p.coff = Sk - 1;
  }
  p.kps = pl.kps;
  p.nrb = pl.nrb;
  p.nrb_m = 0xffffffffu / (uint32_t)pl.nrb;
  p.hkv_m = 0xffffffffu / (uint32_t)Hkv;
  p.zmax = pl.zmax;
  p.zmax_m = 0xffffffffu / (uint32_t)std::max(pl.zmax, 1);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.q_sb = vq.sb, p.q_ss = vq.ss, p.q_sh = vq.sh;
  p.k_sb = vk.sb, p.k_ss = vk.ss, p.k_sh = vk.sh;
  p.v_sb = vv.sb, p.v_ss = vv.ss, p.v_sh = vv.sh;
  p.o_sb = vo.sb, p.o_ss = vo.ss, p.o_sh = vo.sh;
  if (pl.launch.split) {
    Workspace ws;
    if (where == Scratch::kStatic) {
      if (pl.ws_bytes > fa::kStaticScratchBytes) return FA_ERR_SCRATCH;
      if (fa::static_scratch(&ws.ptr) != hipSuccess) return FA_ERR_LAUNCH;
      ws.bytes = fa::kStaticScratchBytes;
    } else {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
      std::lock_guard<std::mutex> lock(g_ws_mu);
      ws = g_ws[dev];
    }
    if (ws.ptr == nullptr || ws.bytes < pl.ws_bytes || !aligned(ws.ptr, 256)) return FA_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws.ptr);
    p.ws_o = reinterpret_cast<float*>(base);
    p.ws_ml = reinterpret_cast<float*>(base + pl.ws_o_bytes);
  }
  const hipError_t e = fa::launch_fwd(p, pl.launch, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t padded_ws_bytes(const Plan& pl) { return pl.launch.split ? pl.ws_bytes : 0; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int code) {
  switch (code) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes or strides (need all sizes >= 1, Hq % Hkv == 0, offsets within 32 bits, non-negative strides, key rows and output rows that do not overlap)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported head_dim (64, 72, 256), element type, or kernel variant";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: q/k/v/out must be 16-byte aligned with strides in multiples of 8 elements, lse/seqused_k 4-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: split-KV path needs a registered workspace of fa_fwd_workspace_bytes() bytes";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime reported an error";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: out or lse overlaps an input (q, k, v, seqused_k, cu_seqlens) or each other";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: fa_fwd_static: this shape's split-KV partials exceed the 8 MiB static scratch (use fa_fwd with a registered workspace)";
    default: return "FA_ERR_UNKNOWN: unknown status code";
  }
}

size_t fa_fwd_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal) {
  if (check_shape(B, Sq, Sk, Hq, Hkv, D, causal) != FA_OK) return 0;
  return padded_ws_bytes(default_plan(B, Sq, Sk, Hq, Hkv, D, causal));
}

size_t fa_fwd_variant_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal, int qt, int nw,
                                      int kw, int bn, int nst, int kps) {
  if (check_shape(B, Sq, Sk, Hq, Hkv, D, causal) != FA_OK) return 0;
  Plan pl;
  if (variant_plan(pl, B, Sq, Sk, Hq, Hkv, D, causal, qt, nw, kw, bn, nst, kps) != FA_OK) return 0;
  return padded_ws_bytes(pl);
}

int fa_set_workspace(void* dev_ptr, size_t bytes) {
  if (dev_ptr == nullptr && bytes > 0) return FA_ERR_NULL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  g_ws[dev].ptr = dev_ptr;
  g_ws[dev].bytes = dev_ptr ? bytes : 0;
  return FA_OK;
}

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk, int Hq,
           int Hkv, int D, int causal, const int32_t* seqused_k, float scale, hipStream_t stream) {
  int rc = check_args(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale);
  if (rc != FA_OK) return rc;
  const Plan pl = default_plan(B, Sq, Sk, Hq, Hkv, D, causal);
  return run(pl, q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, contiguous(Sq, Hq, D), contiguous(Sk, Hkv, D),
             contiguous(Sk, Hkv, D), contiguous(Sq, Hq, D), seqused_k, scale, stream);
}

int fa_fwd_static(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk,
                  int Hq, int Hkv, int D, int causal, const int32_t* seqused_k, float scale, hipStream_t stream) {
  int rc = check_args(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale);
  if (rc != FA_OK) return rc;
  const Plan pl = default_plan(B, Sq, Sk, Hq, Hkv, D, causal);
  return run(pl, q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, contiguous(Sq, Hq, D), contiguous(Sk, Hkv, D),
             contiguous(Sk, Hkv, D), contiguous(Sq, Hq, D), seqused_k, scale, stream, Packed(), nullptr, nullptr,
             Scratch::kStatic);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk,
                   int Hq, int Hkv, int D, int64_t q_sb, int64_t q_ss, int64_t q_sh, int64_t k_sb, int64_t k_ss,
                   int64_t k_sh, int64_t v_sb, int64_t v_ss, int64_t v_sh, int64_t o_sb, int64_t o_ss,
                   int64_t o_sh, int dtype, int causal, const int32_t* seqused_k, float scale,
                   hipStream_t stream) {
  const View vq{q_sb, q_ss, q_sh}, vk{k_sb, k_ss, k_sh}, vv{v_sb, v_ss, v_sh}, vo{o_sb, o_ss, o_sh};
  const int rc = check_strided(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, vq, vk, vv, vo, dtype, causal, seqused_k,
                               scale);
  if (rc != FA_OK) return rc;
  Plan pl = default_plan(B, Sq, Sk, Hq, Hkv, D, causal);
  pl.launch.dtype = dtype;
  if (!fa::variant_exists(D, pl.launch.qt, pl.launch.nw, pl.launch.kw, pl.launch.bn, pl.launch.nst, dtype))
    return FA_ERR_UNSUPPORTED;
  return run(pl, q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, vq, vk, vv, vo, seqused_k, scale, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int Hq, int Hkv, int D, int dtype, int causal, float scale, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || cu_seqlens_q == nullptr ||
      cu_seqlens_k == nullptr)
    return FA_ERR_NULL;
  if (B < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 || total_q < 1 || total_k < 1 || Hq < 1 || Hkv < 1 || D < 1 ||
      Hq % Hkv != 0 || (causal != 0 && causal != 1))
    return FA_ERR_SHAPE;
  if ((long long)B * Hkv > 65535 || (long long)max_seqlen_q * (Hq / Hkv) > INT32_MAX / 2) return FA_ERR_SHAPE;
  if ((long long)total_q * Hq * D > INT32_MAX || (long long)total_k * Hkv * D > INT32_MAX) return FA_ERR_SHAPE;
  if ((long long)max_seqlen_k * Hkv * D * 2 >= (1ll << 31)) return FA_ERR_SHAPE;
  if (!supported_d(D)) return FA_ERR_UNSUPPORTED;
  if (dtype != fa::kBf16 && dtype != fa::kF16) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_ALIGN;
  if ((lse != nullptr && !aligned(lse, 4)) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)total_q * Hq * D * 2, kb = (size_t)total_k * Hkv * D * 2;
  const size_t cb = (size_t)(B + 1) * sizeof(int32_t);
  if (overlap(out, qb, q, qb) || overlap(out, qb, k, kb) || overlap(out, qb, v, kb) ||
      overlap(out, qb, cu_seqlens_q, cb) || overlap(out, qb, cu_seqlens_k, cb))
    return FA_ERR_ALIAS;
  if (lse != nullptr) {
    const size_t lb = (size_t)Hq * total_q * sizeof(float);
    if (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) || overlap(lse, lb, out, qb) ||
        overlap(lse, lb, cu_seqlens_q, cb) || overlap(lse, lb, cu_seqlens_k, cb))
      return FA_ERR_ALIAS;
  }
  Plan pl = default_plan(B, max_seqlen_q, max_seqlen_k, Hq, Hkv, D, causal);
  pl.launch.dtype = dtype;
  if (!fa::variant_exists(D, pl.launch.qt, pl.launch.nw, pl.launch.kw, pl.launch.bn, pl.launch.nst, dtype))
    return FA_ERR_UNSUPPORTED;
  Packed packed;
  packed.cu_q = cu_seqlens_q;
  packed.cu_k = cu_seqlens_k;
  packed.total_q = total_q;
  packed.total_k = total_k;
  const View vq{0, (long long)Hq * D, D}, vk{0, (long long)Hkv * D, D};
  return run(pl, q, k, v, out, lse, B, max_seqlen_q, max_seqlen_k, Hq, Hkv, vq, vk, vk, vq, nullptr, scale, stream,
             packed);
}

int fa_fwd_nvfp4(const void* q, const void* k, const void* v, void* out_fp4, void* out_sf, float* lse, int B,
                 int Sq, int Sk, int Hq, int Hkv, int D, int causal, const int32_t* seqused_k, float scale,
                 hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out_fp4 == nullptr || out_sf == nullptr) return FA_ERR_NULL;
  int rc = check_shape(B, Sq, Sk, Hq, Hkv, D, causal);
  if (rc != FA_OK) return rc;
  if (D % 16 != 0) return FA_ERR_UNSUPPORTED;  // blocks of 16 would straddle heads
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out_fp4, 4)) return FA_ERR_ALIGN;
  if ((lse != nullptr && !aligned(lse, 4)) || (seqused_k != nullptr && !aligned(seqused_k, 4))) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * Sq * Hq;
  const size_t qb = rows * D * 2, kb = (size_t)B * Sk * Hkv * D * 2, cb = rows * D / 2, sb = rows * D / 16;
  const size_t ub = (size_t)B * sizeof(int32_t);
  if (overlap(out_fp4, cb, q, qb) || overlap(out_fp4, cb, k, kb) || overlap(out_fp4, cb, v, kb) ||
      overlap(out_sf, sb, q, qb) || overlap(out_sf, sb, k, kb) || overlap(out_sf, sb, v, kb) ||
      overlap(out_fp4, cb, out_sf, sb))
    return FA_ERR_ALIAS;
  if (seqused_k != nullptr && (overlap(out_fp4, cb, seqused_k, ub) || overlap(out_sf, sb, seqused_k, ub)))
    return FA_ERR_ALIAS;
  if (lse != nullptr) {
    const size_t lb = rows * sizeof(float);
    if (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
        overlap(lse, lb, out_fp4, cb) || overlap(lse, lb, out_sf, sb) ||
        (seqused_k != nullptr && overlap(lse, lb, seqused_k, ub)))
      return FA_ERR_ALIAS;
  }
  Plan pl = default_plan(B, Sq, Sk, Hq, Hkv, D, causal);
  pl.launch.dtype = fa::kBf16;
  pl.launch.outf = fa::kOutNvfp4;
  if (!fa::nvfp4_variant_exists(pl.launch)) return FA_ERR_UNSUPPORTED;
  return run(pl, q, k, v, nullptr, lse, B, Sq, Sk, Hq, Hkv, contiguous(Sq, Hq, D), contiguous(Sk, Hkv, D),
             contiguous(Sk, Hkv, D), contiguous(Sq, Hq, D), seqused_k, scale, stream, Packed(), out_fp4, out_sf);
}

int fa_fwd_variant(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Sq, int Sk,
                   int Hq, int Hkv, int D, int causal, const int32_t* seqused_k, float scale, int qt, int nw,
                   int kw, int bn, int nst, int kps, hipStream_t stream) {
  int rc = check_args(q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, D, causal, seqused_k, scale);
  if (rc != FA_OK) return rc;
  Plan pl;
  rc = variant_plan(pl, B, Sq, Sk, Hq, Hkv, D, causal, qt, nw, kw, bn, nst, kps);
  if (rc != FA_OK) return rc;
  return run(pl, q, k, v, out, lse, B, Sq, Sk, Hq, Hkv, contiguous(Sq, Hq, D), contiguous(Sk, Hkv, D),
             contiguous(Sk, Hkv, D), contiguous(Sq, Hq, D), seqused_k, scale, stream);
}

int fa_fwd_plan(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal, int* qt, int* nw, int* kw, int* bn,
                int* nst, int* kps) {
  int rc = check_shape(B, Sq, Sk, Hq, Hkv, D, causal);
  if (rc != FA_OK) return rc;
  if (qt == nullptr || nw == nullptr || kw == nullptr || bn == nullptr || nst == nullptr || kps == nullptr)
    return FA_ERR_NULL;
  const Plan pl = default_plan(B, Sq, Sk, Hq, Hkv, D, causal);
  *qt = pl.launch.qt;
  *nw = pl.launch.nw;
  *kw = pl.launch.kw;
  *bn = pl.launch.bn;
  *nst = pl.launch.nst;
  *kps = pl.kps;
  return FA_OK;
}

}  // extern "C"
