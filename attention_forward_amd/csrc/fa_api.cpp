// C ABI of the fused attention forward library (declared in include/fa.h).
//
// This file holds the host side only: argument checks, the choice between
// the single-pass and the split-KV kernels, the per-device workspace
// registry, and the launch.  It never touches device memory: seqused_k is
// read only by the kernels.  Checks run before any HIP call, so every error
// path works without a GPU (the failure convention of the pages: explicit
// errors, never an implicit fallback -- "pi05_thor_decoder_fp4_e2e.md",
// section "Implemented Path"; probe before capture -- "GROOT N1.7 update",
// section "Shared-code changes").

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kSplitMinWorkgroups = 64;  // below this many single-pass workgroups, split the keys
constexpr int kSplitMinKeys = 256;       // ... but only when the key buffer is longer than this

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
Workspace g_ws[kMaxDevices];
std::mutex g_ws_mu;

bool supported_d(int D) { return D == 64 || D == 72 || D == 256; }

struct Plan {
  fa::LaunchPlan launch;
  int Mp = 0;
  int kps = 0;
  size_t ws_bytes = 0;
  size_t ws_o_bytes = 0;
};

// Shape-only planning: the same inputs always give the same kernel, tile and
// split, independent of the device-side seqused_k values.
Plan make_plan(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal) {
  Plan pl;
  const int g = Hq / Hkv;
  pl.Mp = Sq * g;
  pl.launch.D = D;
  pl.launch.causal = causal != 0;
  pl.launch.nsplit = 0;
  const long long rows_wg = fa::plan_rows_per_wg(D);
  const long long wgs = (pl.Mp + rows_wg - 1) / rows_wg * (long long)B * Hkv;
  if (!causal && wgs < kSplitMinWorkgroups && Sk > kSplitMinKeys) {
    pl.kps = fa::plan_block_keys(D);
    pl.launch.nsplit = (Sk + pl.kps - 1) / pl.kps;
    const size_t rows = (size_t)pl.launch.nsplit * B * Hkv * pl.Mp;
    pl.ws_o_bytes = (rows * D * sizeof(float) + 255) / 256 * 256;
    pl.ws_bytes = pl.ws_o_bytes + rows * 2 * sizeof(float);
  }
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
  if (!supported_d(D)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int code) {
  switch (code) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes (need all >= 1, Hq % Hkv == 0, 32-bit element counts)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported head_dim (64, 72, 256) or causal with Sq != Sk or with seqused_k";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: q/k/v/out must be 16-byte aligned, lse/seqused_k 4-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: split-KV path needs a registered workspace of fa_fwd_workspace_bytes() bytes";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime reported an error";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: out or lse overlaps an input";
    default: return "FA_ERR_UNKNOWN: unknown status code";
  }
}

size_t fa_fwd_workspace_bytes(int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal) {
  if (check_shape(B, Sq, Sk, Hq, Hkv, D, causal) != FA_OK) return 0;
  return make_plan(B, Sq, Sk, Hq, Hkv, D, causal).ws_bytes;
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

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int B, int Sq, int Sk, int Hq, int Hkv, int D, int causal,
           const int32_t* seqused_k, float scale, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return FA_ERR_NULL;
  int rc = check_shape(B, Sq, Sk, Hq, Hkv, D, causal);
  if (rc != FA_OK) return rc;
  if (causal && (Sq != Sk || seqused_k != nullptr)) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_ALIGN;
  if ((lse != nullptr && !aligned(lse, 4)) || (seqused_k != nullptr && !aligned(seqused_k, 4)))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)B * Sq * Hq * D * 2, kb = (size_t)B * Sk * Hkv * D * 2;
  if (overlap(out, qb, q, qb) || overlap(out, qb, k, kb) || overlap(out, qb, v, kb)) return FA_ERR_ALIAS;
  if (lse != nullptr) {
    const size_t lb = (size_t)B * Hq * Sq * sizeof(float);
    if (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
        overlap(lse, lb, out, qb))
      return FA_ERR_ALIAS;
  }

  const Plan pl = make_plan(B, Sq, Sk, Hq, Hkv, D, causal);
  fa::FwdParams p{};
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
  p.Mp = pl.Mp;
  p.kps = pl.kps;
  p.scale_log2 = scale * 1.4426950408889634f;

  if (pl.launch.nsplit > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    Workspace ws;
    {
      std::lock_guard<std::mutex> lock(g_ws_mu);
      ws = g_ws[dev];
    }
    if (ws.ptr == nullptr || ws.bytes < pl.ws_bytes || !aligned(ws.ptr, 256)) return FA_ERR_WORKSPACE;
    p.ws_o = static_cast<float*>(ws.ptr);
    p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + pl.ws_o_bytes);
  }

  const hipError_t e = fa::launch_fwd(p, pl.launch, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
