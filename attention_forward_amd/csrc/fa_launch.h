// Internal interface between the C ABI (fa_api.cpp) and the gfx950 kernels
// (fa_kernels.hip).  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Everything a forward launch needs, by value (kernel argument).
struct FwdParams {
  const uint16_t* q;       // (batch, position, head, head_dim) view, 16-bit elements
  const uint16_t* k;       // (batch, key, kv head, head_dim) view
  const uint16_t* v;       // (batch, key, kv head, head_dim) view
  uint16_t* out;           // (batch, position, head, head_dim) view, written
  // NVFP4 output instead of out (the NVFP4 variants): per (batch, position,
  // head) row, contiguous, D/2 bytes of E2M1 pairs and D/16 UE4M3 scales.
  uint8_t* fp4_out;
  uint8_t* fp4_sf;
  float* lse;              // [B, Hq, Sq] fp32 contiguous, or null
  const int32_t* seqused;  // [B] int32 on the device, or null
  // Packed variable-length batch (both null otherwise): B + 1 offsets each,
  // on the device, of the sequences along the token dimension of q / out
  // and of k / v (whose batch strides are then 0).
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;    // token rows of q / out and of k / v (packed batch)
  long long lse_hs;        // lse elements between heads: Sq, or total_q for a packed batch
  long long lse_bs;        // lse elements between batch entries: Hq * Sq, or 0 for a packed batch
  // Split-KV workspace (split variants only).  Partial rows are indexed
  // ((bh * nrb + row_block) * zmax + split) * rows_per_block + row_in_block.
  float* ws_o;             // partial O / l, fp32, D per partial row
  float* ws_ml;            // partial (m in log2 units, l), fp32 pairs
  int B, Sq, Sk, Hq, Hkv;
  int g;                   // Hq / Hkv
  uint32_t g_m;            // floor((2^32 - 1) / g), multiplier for udiv
  int Mp;                  // packed rows per (batch, kv head) = Sq * g
  int coff;                // Sk - Sq: causal diagonal offset of the full key buffer (grid planning)
  int kps;                 // keys per split (multiple of the key tile), split variants only
  int nrb;                 // row blocks per (batch, kv head)
  uint32_t nrb_m, hkv_m;   // floor((2^32 - 1) / nrb) and floor((2^32 - 1) / Hkv), multipliers for udiv
  int zmax;                // most splits of any row block
  uint32_t zmax_m;         // floor((2^32 - 1) / zmax) (split variants), multiplier for udiv
  float scale_log2;        // scale * log2(e)
  // Element strides of the views (batch, sequence, head); head_dim is
  // contiguous.  Contiguous BSHD: (S*H*D, H*D, D).
  long long q_sb, q_ss, q_sh;
  long long k_sb, k_ss, k_sh;
  long long v_sb, v_ss, v_sh;
  long long o_sb, o_ss, o_sh;
};

enum ElemType { kBf16 = 0, kF16 = 1 };
enum OutFormat { kOutElem = 0, kOutNvfp4 = 1 };  // out in the element type, or NVFP4

struct LaunchPlan {
  int D;
  int qt;                  // rows per wave / 16
  int nw;                  // waves per workgroup
  int kw;                  // waves that split the keys of the same rows (1: waves own different rows)
  int bn;                  // keys per tile
  int nst;                 // K/V tile stages in LDS
  bool causal;
  bool split;
  int nsplit;              // non-causal split count (grid.z)
  int dtype;               // ElemType of q, k, v and out
  int outf;                // OutFormat of the result
};

constexpr int kComputeUnits = 256;  // MI355X

// Device-resident split-KV scratch of fa_fwd_static (one array per GPU,
// in fa_kernels.hip): its size, and its address on the current device.
constexpr size_t kStaticScratchBytes = 8u << 20;
hipError_t static_scratch(void** ptr);

bool variant_exists(int D, int qt, int nw, int kw, int bn, int nst, int dtype);
bool nvfp4_variant_exists(const LaunchPlan& plan);
hipError_t launch_fwd(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream);

}  // namespace fa
