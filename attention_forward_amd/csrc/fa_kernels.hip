// Fused attention forward for gfx950 (MI355X): out = softmax(scale*Q*K^T + mask)*V
// together with the per-row natural-log log-sum-exp.
//
// The operation and its outputs follow the "flashrt/fa4-cute-runtime" card
// (section "Functions": the forward returns (out, lse); the padded
// fixed-shape example: a device-side seqused_k and pack_gqa).  Masked keys
// get probability exactly zero and are never read from memory, as in the
// seqused attention passage of "pi05_thor_decoder_fp4_e2e.md" (section
// "Fused GeGLU FFN in the Decoder"), so no -inf pre-fill exists anywhere.
//
// Kernel structure (one workgroup = NW wavefronts of 64 lanes):
//  * GQA packing: the g = Hq/Hkv query heads that read one K/V head are
//    folded into the row dimension.  Packed row r of (batch b, kv head hk)
//    is query position r / g of head hk*g + r % g, so one K/V tile staged in
//    LDS serves every head of the group.
//  * Each wave owns 16*QT packed rows.  The contraction is written
//    transposed, S^T = K * Q^T and O^T = V^T * P^T, with the bf16 MFMA
//    v_mfma_f32_16x16x32_bf16.  In the 16x16 accumulator layout lane l holds
//    column l%16, so every lane owns one query row: the softmax statistics
//    live in that lane, the O^T rescale needs no data movement, and the
//    S^T accumulator is already the P^T operand of the second MFMA.
//  * K tiles sit row-major in LDS (padded rows, conflict-free 16-byte
//    reads).  V tiles are written transposed (d-major), with keys permuted
//    inside each 32-key block to match the order P^T comes out of the S^T
//    accumulators, and an XOR swizzle of 16-byte chunks per row.
//  * Online softmax in base 2: t = s*scale*log2(e); running max m and sum l
//    per row; O^T is rescaled by exp2(m_old - m_new) per K/V tile.
//  * Masking touches only the tile that crosses the valid length and the
//    causal diagonal tiles; keys at or past the valid length are never
//    loaded and their V rows in LDS are zero, so padding (even inf/nan)
//    cannot reach an accumulator.
//  * Split-KV variant: blockIdx.z picks a key range; the partial (m, l,
//    O/l) goes to a workspace and a second kernel merges the splits in
//    fixed order (deterministic; no float atomics).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

static constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float wave_max_groups(float x) {
  // max over lanes l, l^16, l^32, l^48 (the four 16-lane rows holding one column)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Position of key kr (0..BN-1) inside the transposed V row.  Within each
// 32-key block, slot 8*grp + e holds the key that the S^T accumulators give
// lane group grp in element e of the P^T operand: e < 4 -> key 4*grp + e of
// the first 16-key M-tile, e >= 4 -> key 16 + 4*grp + (e - 4) of the second.
__device__ __forceinline__ int vt_slot(int kr) {
  const int blk = kr >> 5, kb = kr & 31;
  const int half = kb >> 4, w = kb & 15;
  return blk * 32 + (w >> 2) * 8 + (w & 3) + 4 * half;
}

// XOR swizzle of the 16-byte chunk index inside a transposed-V row.
template <int BN>
__device__ __forceinline__ int vt_swz(int d) {
  constexpr int kChunks = BN / 8;
  return (d ^ (d >> 3)) & (kChunks - 1);
}

template <int D, int QT, int NW, int BN, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(NW * 64)
fwd_kernel(const FwdParams p) {
  constexpr int DP = (D + 31) / 32 * 32;  // head dim padded to the MFMA K step
  constexpr int KC = DP / 32;             // K steps of S^T = K * Q^T
  constexpr int DT = (D + 15) / 16;       // 16-row tiles of O^T
  constexpr int KSTR = DP + 8;            // K row stride in LDS (elements)
  constexpr int VSTR = BN;                // transposed-V row stride (elements)
  constexpr int MT = BN / 16;             // 16-key M tiles of S^T
  constexpr int KVC = BN / 32;            // 32-key K steps of O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int NT = NW * 64;
  constexpr int ROWS_WG = NW * 16 * QT;
  static_assert(D % 8 == 0 && BN % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DT * 16 * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int bh = blockIdx.y;
  const int b = bh / p.Hkv, hk = bh - b * p.Hkv;
  const int g = p.g;
  const int row0 = blockIdx.x * ROWS_WG;
  const int rw0 = row0 + wave * 16 * QT;

  int nvalid = p.Sk;
  if (p.seqused != nullptr) nvalid = min(max(p.seqused[b], 0), p.Sk);
  int kbeg = 0, kend = nvalid;
  if constexpr (SPLIT) {
    kbeg = blockIdx.z * p.kps;
    kend = min(kbeg + p.kps, nvalid);
  }
  if constexpr (CAUSAL) {
    const int rlast = min(row0 + ROWS_WG, p.Mp) - 1;
    kend = min(kend, rlast / g + 1);
  }

  // Q^T fragments (B operand of S^T): lane (col, grp) holds row rw0+16t+col,
  // head-dim elements 32c + 8grp .. +7.
  bf16x8_t qf[QT][KC];
  int srow[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int r = rw0 + 16 * t + col;
    const bool ok = r < p.Mp;
    const int s = ok ? r / g : 0;
    const int hh = ok ? r - s * g : 0;
    srow[t] = ok ? s : -1;
    const uint16_t* qp = p.q + ((size_t)(b * p.Sq + s) * p.Hq + hk * g + hh) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int d0 = 32 * c + 8 * grp;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (ok && d0 < D) x = ldg16(qp + d0);
      qf[t][c] = as_bf16x8(x);
    }
  }
  // The wave's smallest and largest query position (causal tile skipping).
  const int s_lo = min(rw0, p.Mp - 1) / g;
  const int s_hi = (min(rw0 + 16 * QT, p.Mp) - 1) / g;
  const bool wave_active = rw0 < p.Mp;

  // Zero the head-dim padding columns of the K tile once (D = 72 -> 96).
  if constexpr (DP > D) {
    constexpr int PADC = (DP - D) / 8;
    for (int i = tid; i < BN * PADC; i += NT) {
      const int kr = i / PADC, pc = i - kr * PADC;
      *reinterpret_cast<u32x4_t*>(&Ks[kr * KSTR + D + 8 * pc]) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  f32x4_t oacc[DT][QT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int t = 0; t < QT; ++t) oacc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }
  const float c2 = p.scale_log2;
  const size_t kv_base = ((size_t)b * p.Sk * p.Hkv + hk) * D;
  const size_t kv_rstride = (size_t)p.Hkv * D;

  for (int kt = kbeg; kt < kend; kt += BN) {
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < BN * CPR; i += NT) {
      const int kr = i / CPR, ch = i - kr * CPR;
      const int j = kt + kr;
      u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (j < kend) {
        const size_t off = kv_base + (size_t)j * kv_rstride + 8 * ch;
        kx = ldg16(p.k + off);
        vx = ldg16(p.v + off);
      }
      *reinterpret_cast<u32x4_t*>(&Ks[kr * KSTR + 8 * ch]) = kx;
      const int slot = vt_slot(kr);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * ch + e;
        const uint32_t word = vx[e >> 1];
        const uint16_t val = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
        const int pchunk = (slot >> 3) ^ vt_swz<BN>(d);
        Vt[d * VSTR + pchunk * 8 + (slot & 7)] = val;
      }
    }
    __syncthreads();

    if (!wave_active) continue;
    if constexpr (CAUSAL) {
      if (kt > s_hi) continue;  // whole tile above the diagonal for this wave
    }

    // S^T = K * Q^T : lane (col, grp) gets query col, keys 16mt + 4grp + r.
    f32x4_t sacc[MT][QT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < QT; ++t) sacc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8_t kf = as_bf16x8(
            *reinterpret_cast<const u32x4_t*>(&Ks[(16 * mt + col) * KSTR + 32 * c + 8 * grp]));
#pragma unroll
        for (int t = 0; t < QT; ++t)
          sacc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t][c], sacc[mt][t], 0, 0, 0);
      }
    }

    const bool need_mask = (kt + BN > kend) || (CAUSAL && kt + BN - 1 > s_lo);
    uint32_t pk[KVC][QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sacc[mt][t][r] * c2;
          if (need_mask) {
            const int key = kt + 16 * mt + 4 * grp + r;
            bool ok = key < kend;
            if constexpr (CAUSAL) ok = ok && key <= srow[t];
            x = ok ? x : -INFINITY;
          }
          sacc[mt][t][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = wave_max_groups(mx);
      const float m_new = fmaxf(m_run[t], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_use);
      m_run[t] = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sacc[mt][t][r] - m_use);
          sacc[mt][t][r] = pv;
          lsum += pv;
        }
      l_run[t] = l_run[t] * alpha + lsum;
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i][t] *= alpha;
#pragma unroll
      for (int kc = 0; kc < KVC; ++kc) {
        pk[kc][t][0] = pack_bf16x2(sacc[2 * kc][t][0], sacc[2 * kc][t][1]);
        pk[kc][t][1] = pack_bf16x2(sacc[2 * kc][t][2], sacc[2 * kc][t][3]);
        pk[kc][t][2] = pack_bf16x2(sacc[2 * kc + 1][t][0], sacc[2 * kc + 1][t][1]);
        pk[kc][t][3] = pack_bf16x2(sacc[2 * kc + 1][t][2], sacc[2 * kc + 1][t][3]);
      }
    }

    // O^T += V^T * P^T : lane (col, grp) gets query col, head-dim 16dt + 4grp + r.
#pragma unroll
    for (int kc = 0; kc < KVC; ++kc) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + col;
        const int pchunk = (4 * kc + grp) ^ vt_swz<BN>(d);
        const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&Vt[d * VSTR + pchunk * 8]));
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          const u32x4_t pw = {pk[kc][t][0], pk[kc][t][1], pk[kc][t][2], pk[kc][t][3]};
          oacc[dt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, as_bf16x8(pw), oacc[dt][t], 0, 0, 0);
        }
      }
    }
  }

  if (!wave_active) return;

#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float l = wave_sum_groups(l_run[t]);
    const int r = rw0 + 16 * t + col;
    if (r >= p.Mp) continue;
    const int s = r / g, hh = r - s * g;
    const float inv = (l > 0.f) ? 1.0f / l : 0.f;
    if constexpr (!SPLIT) {
      uint16_t* op = p.out + ((size_t)(b * p.Sq + s) * p.Hq + hk * g + hh) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        if (d < D) {
          u32x2_t w = {pack_bf16x2(oacc[dt][t][0] * inv, oacc[dt][t][1] * inv),
                       pack_bf16x2(oacc[dt][t][2] * inv, oacc[dt][t][3] * inv)};
          *reinterpret_cast<u32x2_t*>(op + d) = w;
        }
      }
      if (p.lse != nullptr && grp == 0) {
        const float lse = (l > 0.f) ? (m_run[t] + __log2f(l)) * kLn2 : -INFINITY;
        p.lse[((size_t)b * p.Hq + hk * g + hh) * p.Sq + s] = lse;
      }
    } else {
      // Partial for this key range: normalised O, the running max (log2
      // units) and the row sum.  An empty range stores l = 0.
      const size_t prow = ((size_t)blockIdx.z * gridDim.y + bh) * p.Mp + r;
      float* po = p.ws_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        if (d < D) {
          f32x4_t w = oacc[dt][t] * inv;
          *reinterpret_cast<f32x4_t*>(po + d) = w;
        }
      }
      if (grp == 0) {
        p.ws_ml[2 * prow] = m_run[t];
        p.ws_ml[2 * prow + 1] = l;
      }
    }
  }
}

// Merge the split partials of one packed row, in split order:
//   M = max_s m_s over non-empty splits, w_s = l_s * 2^(m_s - M),
//   out = sum_s w_s * Ohat_s / sum_s w_s,  lse = ln2 * (M + log2 sum_s w_s).
// One thread per (packed row, 8 head-dim elements).
template <int D>
__global__ void __launch_bounds__(256)
combine_kernel(const FwdParams p, int nsplit, int BH) {
  constexpr int CPR = D / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)BH * p.Mp * CPR;
  if (i >= total) return;
  const int ch = (int)(i % CPR);
  const long long rr = i / CPR;
  const int r = (int)(rr % p.Mp);
  const int bh = (int)(rr / p.Mp);
  const int b = bh / p.Hkv, hk = bh - b * p.Hkv;
  const int g = p.g;
  const size_t split_stride = (size_t)BH * p.Mp;

  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) {
    const size_t prow = s * split_stride + rr;
    const float l = p.ws_ml[2 * prow + 1];
    if (l > 0.f) M = fmaxf(M, p.ws_ml[2 * prow]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const size_t prow = s * split_stride + rr;
    const float l = p.ws_ml[2 * prow + 1];
    if (!(l > 0.f)) continue;
    const float w = l * __builtin_amdgcn_exp2f(p.ws_ml[2 * prow] - M);
    L += w;
    const f32x4_t* po = reinterpret_cast<const f32x4_t*>(p.ws_o + prow * D + 8 * ch);
    const f32x4_t a0 = po[0], a1 = po[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += w * a0[e];
      acc[4 + e] += w * a1[e];
    }
  }
  const int sq = r / g, hh = r - sq * g;
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<u32x4_t*>(p.out + ((size_t)(b * p.Sq + sq) * p.Hq + hk * g + hh) * D + 8 * ch) = o;
  if (ch == 0 && p.lse != nullptr) {
    const float lse = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
    p.lse[((size_t)b * p.Hq + hk * g + hh) * p.Sq + sq] = lse;
  }
}

template <int D, int QT, int NW, int BN, bool CAUSAL, bool SPLIT>
static hipError_t launch_one(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  constexpr int ROWS_WG = NW * 16 * QT;
  dim3 grid((p.Mp + ROWS_WG - 1) / ROWS_WG, p.B * p.Hkv, SPLIT ? plan.nsplit : 1);
  hipLaunchKernelGGL((fwd_kernel<D, QT, NW, BN, CAUSAL, SPLIT>), grid, dim3(NW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !SPLIT) return e;
  const long long threads = (long long)p.B * p.Hkv * p.Mp * (D / 8);
  dim3 cgrid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL((combine_kernel<D>), cgrid, dim3(256), 0, stream, p, plan.nsplit, p.B * p.Hkv);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  constexpr int QT = 2, NW = 4, BN = 64;
  if (plan.causal) return launch_one<D, QT, NW, BN, true, false>(p, plan, stream);
  if (plan.nsplit > 0) return launch_one<D, QT, NW, BN, false, true>(p, plan, stream);
  return launch_one<D, QT, NW, BN, false, false>(p, plan, stream);
}

int plan_rows_per_wg(int /*D*/) { return 4 * 16 * 2; }
int plan_block_keys(int /*D*/) { return 64; }

hipError_t launch_fwd(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  switch (plan.D) {
    case 64: return launch_d<64>(p, plan, stream);
    case 72: return launch_d<72>(p, plan, stream);
    case 256: return launch_d<256>(p, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
