// Internal interface between the C ABI (fa_api.cpp) and the gfx950 kernels
// (fa_kernels.hip).  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Everything a forward launch needs, by value (kernel argument).
struct FwdParams {
  const uint16_t* q;   // [B, Sq, Hq, D] bf16
  const uint16_t* k;   // [B, Sk, Hkv, D] bf16
  const uint16_t* v;   // [B, Sk, Hkv, D] bf16
  uint16_t* out;       // [B, Sq, Hq, D] bf16
  float* lse;          // [B, Hq, Sq] fp32 or null
  const int32_t* seqused;  // [B] int32 on the device, or null
  float* ws_o;         // split partials: [nsplit, B*Hkv, Mp, D] fp32
  float* ws_ml;        // split partials: [nsplit, B*Hkv, Mp, 2] fp32 (m, l)
  int B, Sq, Sk, Hq, Hkv;
  int g;               // Hq / Hkv
  int Mp;              // packed rows per (batch, kv head) = Sq * g
  int kps;             // keys per split (multiple of the key tile), split path only
  float scale_log2;    // scale * log2(e)
};

struct LaunchPlan {
  int D;
  bool causal;
  int nsplit;          // 0: single pass; >= 1: split-KV path with that many splits
};

// Tile geometry the host needs for planning.
int plan_rows_per_wg(int D);
int plan_block_keys(int D);

hipError_t launch_fwd(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream);

}  // namespace fa
