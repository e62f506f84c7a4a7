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
//  * Each wave owns 16*QT packed rows; all waves share the K/V tiles.  The
//    contractions are written transposed, S^T = K * Q^T and O^T = V^T * P^T,
//    on v_mfma_f32_16x16x32_bf16.  In the 16x16 accumulator layout lane l
//    holds column l%16, so every lane owns one query row: its softmax
//    statistics stay in the lane, the O^T rescale needs no data movement,
//    and the S^T accumulator is already the P^T operand of the second MFMA.
//  * K and V tiles are stored row-major in LDS with padded row strides
//    (K rows 16 bytes apart modulo 128, V rows 32 bytes apart modulo 128)
//    so that the fragment reads are free of bank conflicts and every read
//    address is one per-lane base plus a compile-time offset.  The tiles are
//    filled by buffer loads that write LDS directly (no VGPR staging); rows
//    at or past the end of the key range fall outside the buffer range and
//    arrive as zeros, so padding keys are never read from memory.  The V^T
//    operand is read with ds_read_b64_tr_b16, which transposes 16-bit data
//    on the way out of LDS.
//  * A ring of NST K/V stages: the loads of the next NST-1 tiles are in
//    flight while one tile is computed.
//  * Online softmax in base 2: t = s*scale*log2(e), running max m and sum
//    l per row, row reductions across the four 16-lane rows with
//    v_permlane16/32_swap.  The rescale of O is lazy: the running max is
//    only moved (and O, l rescaled) when a row's max grows by more than 2^8,
//    otherwise exp2 is taken against the stale max (values stay <= 256).
//  * Masking touches only the tile that crosses the end of the key range
//    and the causal diagonal tiles.
//  * Split-KV: several workgroups share one block of rows and each takes a
//    key range.  Each writes its partial (O/l, m, l) to the workspace; a
//    second, fully parallel kernel on the same stream merges the partials of
//    every row in fixed split order (deterministic, no float atomics).
//  * Causal: row blocks are dispatched heaviest first; with splitting, the
//    key range [0, last position of the block] is cut into fixed chunks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ----------------------------------------------------- static split scratch
// The split-KV partials of fa_fwd_static live here instead of in a
// caller-registered workspace, for callers that cannot allocate.  Each GPU
// the library runs on holds its own copy for the life of the process.  In
// host code the name `scratch` is only a host-side stand-in: the device
// address of the current GPU's copy comes from hipGetSymbolAddress, taken
// once per device and kept.  Nothing in it has to start at zero: every
// partial the merge kernel reads is written earlier by the same call.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}


template <int D, int QT, int NW, int BN, int NST, int KG, bool CAUSAL, bool SPLIT, int DTY, int OUTF>
__global__ void __launch_bounds__(NW * KG * 64, 1)
fwd_kernel(const FwdParams p) {
  using G = Geo<D, QT, NW, BN, DTY>;  // geometry of one key group: NW waves on different rows
  static_assert(NST >= 2, "at least double buffering");
  static_assert(KG == 1 || (KG == 2 && NST == 2), "two key groups run the two-stage loop");
  static_assert(OUTF == kOutElem || D % 16 == 0, "NVFP4 blocks of 16 stay inside a head");
  static_assert(KG * NST * G::STAGE_B + (G::TRASH ? NW * KG * 1024 : 16) <= 160 * 1024, "LDS of one workgroup");
  __shared__ __attribute__((aligned(16))) uint8_t stage[KG * NST * G::STAGE_B];
  __shared__ __attribute__((aligned(16))) uint8_t trash[G::TRASH ? NW * KG * 1024 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // KG key groups of NW waves: group kg takes key tiles kg, kg+KG, ... of the
  // block's range through its own stage ring, wave w of each group owns the
  // same rows, and the groups' partial results are merged at the end.
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level addresses stay scalar
  const int kg = KG > 1 ? wid / NW : 0;
  const int wave = wid - kg * NW;                            // row wave within the group
  const int gtid = tid - kg * NW * 64;                       // thread within the group
  const int col = lane & 15, grp = lane >> 4;
  pin_params(p);
  int bh, rb_x;
  if constexpr (CAUSAL || SPLIT) {
    bh = blockIdx.y;
    rb_x = blockIdx.x;
  } else {
    xcd_block(p, bh, rb_x);
  }
  const int b = udiv(bh, p.Hkv, p.hkv_m), hk = bh - b * p.Hkv;
  const int g = p.g;

  const Seq sq = seq_of(p, b);
  const int nvalid = sq.nk;
  const int Mp = sq.sq * g;  // packed rows of this batch entry (the grid covers the planned maximum)

  // Which rows and keys this workgroup takes.
  RowBlock blk;
  if constexpr (CAUSAL) {
    int rb, item, kmax;
    if (!causal_item<SPLIT>(p, G::ROWS_WG, g, rb, item, kmax)) return;
    blk.rb = rb;
    blk.z = item;
    blk.kbeg = SPLIT ? item * p.kps : 0;
    blk.kend = SPLIT ? min(blk.kbeg + p.kps, kmax) : kmax;
    // the valid keys, up to the diagonal of the block's last row
    blk.kend = min(min(blk.kend, nvalid), udiv(max(min((rb + 1) * G::ROWS_WG, Mp) - 1, 0), g, p.g_m) + (nvalid - sq.sq) + 1);
  } else {
    blk.rb = rb_x;
    blk.z = SPLIT ? blockIdx.z : 0;
    blk.kbeg = SPLIT ? blk.z * p.kps : 0;
    blk.kend = SPLIT ? min(blk.kbeg + p.kps, nvalid) : nvalid;
  }
  const int row0 = blk.rb * G::ROWS_WG;
  if (row0 >= Mp) return;  // past a shorter sequence of a packed batch: nothing to do
  const int rw0 = row0 + wave * 16 * QT;
  const int kbeg = blk.kbeg, kend = blk.kend;

  typename G::E::v8 qf[QT][G::KC];
  int srow[QT];
  const bool wave_active = rw0 < Mp;
  // Causal: diagonal keys (last attended key) of the wave's first and last
  // rows; the last query lines up with the last valid key.
  const int doff = CAUSAL ? nvalid - sq.sq : 0;
  const int s_lo = udiv(min(rw0, Mp - 1), g, p.g_m) + doff;
  const int s_hi = udiv(min(rw0 + 16 * QT, Mp) - 1, g, p.g_m) + doff;

  f32x4_t oacc[G::DT][QT];
#pragma unroll
  for (int i = 0; i < G::DT; ++i)
#pragma unroll
    for (int t = 0; t < QT; ++t) oacc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }
  const float c2 = p.scale_log2;

  // ---- K/V tile copies.  Buffers start at this (batch, kv head)'s first key
  // and end after key kend - 1, so every key at or past kend reads as zero.
  const uint32_t rstride_k = (uint32_t)(p.k_ss * 2), rstride_v = (uint32_t)(p.v_ss * 2);  // bytes between keys
  const u32x4_t rk = make_rsrc(p.k + view_off(b, sq.k0, hk, p.k_sb, p.k_ss, p.k_sh), (uint32_t)kend * rstride_k);
  const u32x4_t rv = make_rsrc(p.v + view_off(b, sq.k0, hk, p.v_sb, p.v_ss, p.v_sh), (uint32_t)kend * rstride_v);
  // Per-thread source offsets of its slots within a tile: slot P holds row
  // P / (STR/16), chunk P % (STR/16); padding chunks and trash windows read
  // out of range (zeros, no memory access).
  uint32_t voff_k[G::LPT_K], voff_v[G::LPT_V];
#pragma unroll
  for (int j = 0; j < G::LPT_K; ++j) {
    const int P = j * G::NT + gtid;
    const int row = P / (G::KSTR / 16), ch = P - row * (G::KSTR / 16);
    voff_k[j] = (P < G::K_SLOTS && ch < G::CPR) ? row * rstride_k + ch * 16 : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < G::LPT_V; ++j) {
    const int P = j * G::NT + gtid;
    const int row = P / (G::VSTR / 16), ch = P - row * (G::VSTR / 16);
    voff_v[j] = (P < G::V_SLOTS && ch < G::CPR) ? row * rstride_v + ch * 16 : kOutOfRange;
  }
  uint8_t* const gstage = stage + kg * NST * G::STAGE_B;  // this group's stage ring
  const uint32_t lds_stage0 = (uint32_t)(uintptr_t)(lds_void_t*)gstage;
  const uint32_t lds_trash = (uint32_t)(uintptr_t)(lds_void_t*)trash + wid * 1024;
  // The tile's key offset goes into the per-lane offset (not soffset), so
  // the range check sees the full offset; key bytes per batch and head stay
  // below 2^31 (checked on the host), so adding it to kOutOfRange cannot wrap.
  // Group-local tile j holds keys kbeg + (kg + j*KG)*BN ...; it sits in stage j % NST.
  auto issue = [&](int it) __attribute__((always_inline)) {
    const uint32_t st = lds_stage0 + (it % NST) * G::STAGE_B;
    const uint32_t toff_k = (uint32_t)(kbeg + (kg + it * KG) * BN) * rstride_k;
    const uint32_t toff_v = (uint32_t)(kbeg + (kg + it * KG) * BN) * rstride_v;
#pragma unroll
    for (int j = 0; j < G::LPT_K; ++j) {
      const int pbase = j * G::NT + wave * 64;
      const uint32_t dst = (!G::TRASH || pbase < G::K_SLOTS) ? st + pbase * 16 : lds_trash;
      copy16_to_lds(rk, voff_k[j] + toff_k, __builtin_amdgcn_readfirstlane(dst));
    }
#pragma unroll
    for (int j = 0; j < G::LPT_V; ++j) {
      const int pbase = j * G::NT + wave * 64;
      const uint32_t dst = (!G::TRASH || pbase < G::V_SLOTS) ? st + G::K_B + pbase * 16 : lds_trash;
      copy16_to_lds(rv, voff_v[j] + toff_v, __builtin_amdgcn_readfirstlane(dst));
    }
  };

  uint32_t k_lane, v_lane;
  lane_bases<G>(lane, k_lane, v_lane);

  // One K/V tile of the main loop, read from stage `st`.
  auto compute_tile = [&](const uint8_t* st, int kt) __attribute__((always_inline)) {
    if (!wave_active) return;
    if constexpr (CAUSAL) {
      if (kt > s_hi) return;  // tile entirely above this wave's diagonal
    }
    f32x4_t sacc[G::MT][QT];
    uint32_t pk[G::KVC][QT][4];
    qk_tile<G, QT>(sacc, qf, st + k_lane, grp);
    softmax_tile<G, QT, CAUSAL>(sacc, pk, m_run, l_run, oacc, srow, kt, kend, s_lo, c2, grp);
    __builtin_amdgcn_sched_barrier(0);
    pv_tile<G, QT>(oacc, pk, st + v_lane);
  };

  // Main loop over a ring of NST K/V stages: tile it sits in stage it % NST
  // and the loads of tiles it+1 .. it+NST-1 are in flight while tile it is
  // computed.  Each tile costs every thread exactly LPT copies, so waiting
  // until at most (NST-2)*LPT copies are outstanding means tile it landed.
  const int ntiles_all = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
  const int ntiles = ntiles_all > kg ? (ntiles_all - kg + KG - 1) / KG : 0;  // this group's tiles
  const int nsteps = (ntiles_all + KG - 1) / KG;                             // loop trips of every group
  // Q^T fragments (B operand of S^T): lane (col, grp) holds packed row
  // rw0 + 16t + col, head-dim elements 32c + 8grp .. +7 (zero past D).
  // Loaded before the first K/V copies, whose issue the memory pipeline
  // paces, so that the Q latency runs under it.
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int r = rw0 + 16 * t + col;
    const bool ok = r < Mp;
    const int s = ok ? udiv(r, g, p.g_m) : 0;
    const int hh = ok ? r - s * g : 0;
    srow[t] = ok ? s + doff : -1;  // causal: the row's diagonal key
    const uint16_t* qp = p.q + view_off(b, sq.q0 + s, hk * g + hh, p.q_sb, p.q_ss, p.q_sh);
#pragma unroll
    for (int c = 0; c < G::KC; ++c) {
      const int d0 = 32 * c + 8 * grp;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (ok && d0 < D) x = ldg16(qp + d0);
      qf[t][c] = G::E::cast(x);
    }
  }
#pragma unroll
  for (int it = 0; it < NST - 1; ++it)
    if (it < ntiles) issue(it);

  // vmcnt(0) as a builtin, so that the compiler knows the Q fragments have
  // landed; the prologue tiles are waited for along with them.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  if constexpr (NST == 2) {
    // Every group makes the same number of trips (the workgroup barrier is
    // shared); a group past its last tile only waits.
    for (int it = 0; it < nsteps; ++it) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // tile it landed (this thread's copies)
      __syncthreads();                            // everyone's copies; the other stage is free
      if (it + 1 < ntiles) issue(it + 1);
      if (it < ntiles) compute_tile(gstage + (it & 1) * G::STAGE_B, kbeg + (kg + it * KG) * BN);
    }
  } else {
    // Software-pipelined loop (three or more stages).  Iteration it issues the
    // copies of tile it+NST-1 into the stage tile it-1 used, then computes
    // S^T of tile it+1 in the same straight-line block as the softmax of
    // tile it (the MFMAs run while the wave issues the softmax VALU work),
    // then O^T += V^T P^T of tile it.  Before the next iteration tile it+2
    // must have landed (its S^T comes next) and every wave must be done
    // with stage it.
    constexpr int kAhead = (NST - 3) * G::LPT;  // copies allowed in flight after tile it+2
    static_assert(kAhead < 64, "vmcnt holds at most 63");
    __syncthreads();  // the prologue tiles are visible to every wave
    f32x4_t s_cur[G::MT][QT];
    bool act = wave_active && ntiles > 0;
    if constexpr (CAUSAL) act = act && kbeg <= s_hi;
    if (act) qk_flat<G, QT>(s_cur, qf, stage + k_lane);
    // Byte offsets of the stages of tiles it and it+1, rotated explicitly.
    int off_cur = 0, off_nxt = G::STAGE_B;
    for (int it = 0; it < ntiles; ++it) {
      if (it + NST - 1 < ntiles) issue(it + NST - 1);
      const int kt = kbeg + it * BN;
      act = wave_active;
      if constexpr (CAUSAL) act = act && kt <= s_hi;  // tiles above the wave's last row are skipped
      if (act) {
        mask_tile<G, QT, CAUSAL>(s_cur, srow, kt, kend, s_lo, grp);
        __builtin_amdgcn_sched_barrier(0);
        // S^T of the next tile (past the last tile the stage holds stale
        // data and the result is never used) overlapped with this tile's
        // softmax, then O^T += V^T P^T of this tile.
        f32x4_t s_nxt[G::MT][QT];
        uint32_t pk[G::KVC][QT][4];
        pipe_tile<G, QT>(s_nxt, s_cur, qf, stage + off_nxt + k_lane, pk, m_run, l_run, oacc, c2);
        __builtin_amdgcn_sched_barrier(0);
        pv_tile<G, QT>(oacc, pk, stage + off_cur + v_lane);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int t = 0; t < QT; ++t) s_cur[mt][t] = s_nxt[mt][t];
      }
      off_cur = off_nxt;
      off_nxt = (off_nxt == (NST - 1) * G::STAGE_B) ? 0 : off_nxt + G::STAGE_B;
      if (it + NST - 1 < ntiles)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAhead));  // tile it+2 landed (this thread's copies)
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __syncthreads();  // everyone's copies; stage it is free
    }
  }

  float l_tot[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) l_tot[t] = group_sum(l_run[t]);

  if constexpr (KG > 1) {
    // ---- merge of the two key groups through LDS: wave w of group 1 stores
    // its O (not yet divided by l) and (m, l) per row; the same lane of wave w
    // of group 0 holds the same elements of the same rows and combines them:
    // M = max of the non-empty m, O = O0 2^(m0-M) + O1 2^(m1-M), l likewise.
    constexpr int OSTR = G::DT * 64 + 16;  // bytes per merged row (padded)
    static_assert(G::ROWS_WG * (OSTR + 8) <= KG * NST * G::STAGE_B, "merge area inside the stages");
    float* mls = reinterpret_cast<float*>(stage + G::ROWS_WG * OSTR);  // [row] (m, l)
    __syncthreads();  // every wave is done with its stages: the LDS becomes the merge area
    if (kg == 1) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int rr = wave * 16 * QT + 16 * t + col;
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt)
          *reinterpret_cast<f32x4_t*>(stage + rr * OSTR + (16 * dt + 4 * grp) * 4) = oacc[dt][t];
        if (grp == 0) *reinterpret_cast<u32x2_t*>(mls + 2 * rr) = u32x2_t{__float_as_uint(m_run[t]), __float_as_uint(l_tot[t])};
      }
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int rr = wave * 16 * QT + 16 * t + col;
      const float m1 = mls[2 * rr], l1 = mls[2 * rr + 1];
      const float m0 = m_run[t], l0 = l_tot[t];
      const float M = fmaxf(l0 > 0.f ? m0 : -INFINITY, l1 > 0.f ? m1 : -INFINITY);
      const float a0 = l0 > 0.f ? __builtin_amdgcn_exp2f(m0 - M) : 0.f;
      const float a1 = l1 > 0.f ? __builtin_amdgcn_exp2f(m1 - M) : 0.f;
      m_run[t] = M;
      l_tot[t] = l0 * a0 + l1 * a1;
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt)
        oacc[dt][t] = oacc[dt][t] * a0 + *reinterpret_cast<const f32x4_t*>(stage + rr * OSTR + (16 * dt + 4 * grp) * 4) * a1;
    }
  }

  if (!wave_active) return;
  if constexpr (!SPLIT) {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int r = rw0 + 16 * t + col;
      if (r >= Mp) continue;
      const int s = udiv(r, g, p.g_m), hh = r - s * g;
      const float l = l_tot[t];
      const float inv = (l > 0.f) ? 1.0f / l : 0.f;
      if constexpr (OUTF == kOutNvfp4) {
        // Block dt is head-dim 16dt .. 16dt+15: four elements in each of the
        // row's four lanes (l, l^16, l^32, l^48), whose amax group_max takes.
        const size_t row = nvfp4_row(p, b, s, hk * g + hh);
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) {
          const f32x4_t x = oacc[dt][t] * inv;
          float div;
          const uint32_t sc = nvfp4_scale(group_max(amax4(x)), div);
          *reinterpret_cast<uint16_t*>(p.fp4_out + row * (D / 2) + 8 * dt + 2 * grp) = (uint16_t)nvfp4_pack4(x, div);
          if (grp == 0) p.fp4_sf[row * (D / 16) + dt] = (uint8_t)sc;
        }
      } else {
        uint16_t* op = p.out + view_off(b, sq.q0 + s, hk * g + hh, p.o_sb, p.o_ss, p.o_sh);
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) {
          const int d = 16 * dt + 4 * grp;
          if (d < D) {
            u32x2_t w = {G::E::pack(oacc[dt][t][0] * inv, oacc[dt][t][1] * inv),
                         G::E::pack(oacc[dt][t][2] * inv, oacc[dt][t][3] * inv)};
            *reinterpret_cast<u32x2_t*>(op + d) = w;
          }
        }
      }
      if (p.lse != nullptr && grp == 0) {
        const float lse = (l > 0.f) ? (m_run[t] + __log2f(l)) * kLn2 : -INFINITY;
        p.lse[sq.lse0 + (long long)(hk * g + hh) * p.lse_hs + s] = lse;
      }
    }
  } else {
    // ---- Partial of this key range: O/l, m (log2 units), l; empty: l = 0.
    // Merged by combine_kernel, launched right after on the same stream.
    const size_t slot_base = ((size_t)bh * p.nrb + blk.rb) * p.zmax;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int rl = wave * 16 * QT + 16 * t + col;  // row within the block
      if (row0 + rl >= Mp) continue;
      const size_t prow = (slot_base + blk.z) * G::ROWS_WG + rl;
      const float l = l_tot[t];
      const float inv = (l > 0.f) ? 1.0f / l : 0.f;
      float* po = p.ws_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        if (d < D) *reinterpret_cast<f32x4_t*>(po + d) = oacc[dt][t] * inv;
      }
      if (grp == 0)
        *reinterpret_cast<u32x2_t*>(p.ws_ml + 2 * prow) = u32x2_t{__float_as_uint(m_run[t]), __float_as_uint(l)};
    }
  }
}

// ------------------------------------------------- key-split workgroup kernel
// All KW waves of a workgroup own the same 16*QT packed rows and split the
// workgroup's key range between them: wave w takes key tiles w, w+KW, ...
// Each wave streams its own K and V tiles into its own LDS buffers (one K
// and one V buffer: the next K tile is loaded during the softmax and PV of
// the current one, the next V tile during the next QK^T), so the main loop
// has no workgroup barrier.  At the end the KW partial results (O, m, l) are
// merged in wave order through LDS.  Compared with fwd_kernel (waves own
// different rows and share tiles), a workgroup covers KW times fewer rows, so
// a small number of rows still fills the chip, while each wave keeps 16*QT
// rows against every K/V byte it reads from LDS.
//
// NST selects the buffer scheme of each wave.  NST == 1: one K and one V
// tile buffer in padded row-major layout; a buffer is refilled after the
// whole tile has been read.  NST == 2 (piecewise refill): the buffers are
// cut into 1 KiB pieces, each the target of one copy instruction, and the
// copy of the next tile's piece is issued as soon as this tile's reads of
// that piece have returned.  A wave then keeps about one tile of K and V in
// flight at all times instead of part of one, which is what the compute
// unit's intake from L2 needs at head dim 256 (its latency is about 1000
// clocks, so streaming at ~56 bytes per clock takes ~56 KiB in flight per
// compute unit).  Pieces, for 32-key tiles:
//   K piece (c, mt): keys 16mt .. 16mt+15, head-dim 32c .. 32c+31, 64 bytes
//     per key; the 16-byte quarter q of key k sits at quarter q ^ (k/4 % 4)
//     of its row, so the 16 keys one fragment read takes at one quarter
//     fall in 16 different bank groups;
//   V piece e: keys 0 .. 31, head-dim 32e .. 32e+31, 64 bytes per key; the
//     16-byte quarter q of key k sits at quarter q ^ 2(k/4 % 2), so the
//     transpose reads of 8 keys at one 16-element column hit 64 different
//     banks.
// Copies of 64-byte row segments run at the full intake rate (32-byte
// segments at about half).
// NST == 3 (ring): the piecewise refill through one buffer per wave whose
// slots take K and V pieces in turn (below), so that a workgroup needs
// 80 KiB of LDS and two run on each compute unit, two waves per SIMD.
template <int D, int QT, int KW, int BN, int NST, bool CAUSAL, bool SPLIT, int DTY, int OUTF>
__global__ void __launch_bounds__(KW * 64, NST == 3 ? 2 : 1)
fwd_ks_kernel(const FwdParams p) {
  using G = Geo<D, QT, 1, BN, DTY>;  // per-wave geometry: one wave issues its own tile copies
  constexpr int ROWS = 16 * QT;
  constexpr bool PIECES = NST >= 2;
  constexpr bool RING = NST == 3;
  pin_params(p);
  static_assert(NST >= 1 && NST <= 3, "buffer scheme");
  static_assert(!G::TRASH, "per-wave tiles must be whole 64-slot windows");
  static_assert(!PIECES || (BN == 32 && D % 32 == 0), "piecewise refill: 32-key tiles, whole 32-element K steps");
  static_assert(!RING || (D == 256 && QT == 2), "ring: 32 rows of head dim 256");
  // LDS: KW per-wave K/V buffers, then the workgroup's Q tile (rows at the K
  // stride, read like K fragments; in the ring scheme unpadded, its 16-byte
  // chunks XOR-swizzled by the row); after the main loop the same memory is
  // the merge area.
  constexpr int K_PIECES = G::KC * G::MT, V_PIECES = G::DT / 2;  // 1 KiB K pieces, 2 KiB V pieces
  constexpr int WAVE_B = RING ? K_PIECES * 1024 : PIECES ? (K_PIECES + 2 * V_PIECES) * 1024 : G::STAGE_B;
  static_assert(!RING || K_PIECES == 2 * V_PIECES, "a ring slot holds either two K pieces or one V piece");
  constexpr int QSTR = RING ? D * 2 : G::KSTR;                     // Q row stride in LDS
  constexpr int Q_INSTR = round_up(ROWS * (QSTR / 16), 64) / 64;  // 1 KiB copies of the Q tile
  constexpr int Q_OFF = KW * WAVE_B;
  // Merge area: wave w's O rows go into its own K/V buffer, so a wave
  // stores them as soon as its own tiles are done.  Rows that are a whole
  // number of 256-byte bank rows are unpadded, their 16-byte chunks
  // XOR-swizzled by the row (chunk c of row r at c ^ (r % 16), which stays
  // inside c's group of 16 chunks); others are padded by 16 bytes.  Either way the 16 rows one store instruction
  // covers, and the rows and chunks one merge read covers, fall in
  // different banks.
  constexpr bool OSWZ = (D * 4) % 256 == 0;
  constexpr int OSTR = OSWZ ? D * 4 : D * 4 + 16;
  constexpr int OROWS = RING ? 16 : ROWS;  // O rows a wave stores per merge pass
  static_assert(OROWS * OSTR <= WAVE_B, "a wave's O rows of one merge pass fit its K/V buffer");
  // (m, l) per row and wave; in the ring scheme in the Q area, which is
  // free once every wave has read its Q fragments
  constexpr int MLS_OFF = RING ? Q_OFF : Q_OFF + Q_INSTR * 1024;
  constexpr int LDS_B = RING ? Q_OFF + Q_INSTR * 1024 : MLS_OFF + KW * ROWS * 8;
  static_assert(!RING || KW * ROWS * 8 <= Q_INSTR * 1024, "ring: (m, l) fit the Q area");
  static_assert(LDS_B <= (RING ? 80 : 160) * 1024, "LDS of one workgroup (ring: two per compute unit)");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level addresses stay scalar
  const int col = lane & 15, grp = lane >> 4;
  int bh = blockIdx.y;
  int rb_nc = blockIdx.x, z_nc = SPLIT ? blockIdx.z : 0;  // non-causal row block and key range
  if constexpr (SPLIT && !CAUSAL) {
    // Items in (bh, key range, row block) order, each XCD taking a
    // contiguous run of them: an XCD's L2 then holds the K/V of about
    // N / 8 / nrb key ranges instead of all of them.
    const int nbh = p.B * p.Hkv;
    const int n = blockIdx.x + p.nrb * (blockIdx.y + nbh * blockIdx.z);  // dispatch order
    const int item = xcd_run(n, p.nrb * nbh * p.zmax);
    const int t = udiv(item, p.nrb, p.nrb_m);
    rb_nc = item - t * p.nrb;
    bh = udiv(t, p.zmax, p.zmax_m);
    z_nc = t - bh * p.zmax;
  }
  const int b = udiv(bh, p.Hkv, p.hkv_m), hk = bh - b * p.Hkv;
  const int g = p.g;

  const Seq sq = seq_of(p, b, false);
  const int Mp = sq.sq * g;  // packed rows of this batch entry (the grid covers the planned maximum)

  RowBlock blk;
  int kmax = 0;
  if constexpr (CAUSAL) {
    int rb, item;
    if (!causal_item<SPLIT, RING>(p, ROWS, g, rb, item, kmax)) return;
    blk.rb = rb;
    blk.z = item;
  } else {
    blk.rb = rb_nc;
    blk.z = z_nc;
  }
  const int row0 = blk.rb * ROWS;
  if (row0 >= Mp) return;  // past a shorter sequence of a packed batch: nothing to do

  // Q tile: packed rows row0 .. row0+ROWS-1, copied once per workgroup
  // (wave w issues copies w, w+KW, ...) into LDS at the K row stride.  The
  // buffer starts at the block's first position; rows past Mp and the row
  // padding read as zeros.
  {
    const int s_first = udiv(row0, g, p.g_m);
    const int s_last = udiv(min(row0 + ROWS, Mp) - 1, g, p.g_m);
    const uint32_t qrow_b = (uint32_t)(p.q_ss * 2), qhead_b = (uint32_t)(p.q_sh * 2);
    const u32x4_t rq = make_rsrc(p.q + view_off(b, sq.q0 + s_first, hk * g, p.q_sb, p.q_ss, p.q_sh),
                                 (uint32_t)(s_last - s_first) * qrow_b + (uint32_t)(g - 1) * qhead_b + D * 2);
    const uint32_t lds_q = (uint32_t)(uintptr_t)(lds_void_t*)(smem + Q_OFF);
    for (int j = wave; j < Q_INSTR; j += KW) {
      const int P = j * 64 + lane;
      const int row = P / (QSTR / 16), sc = P - row * (QSTR / 16);
      const int ch = RING ? (sc ^ (row & 15)) : sc;  // the chunk this LDS slot holds
      const int r = row0 + row;
      uint32_t off = kOutOfRange;
      if (row < ROWS && ch < G::CPR && r < Mp) {
        const int sq = udiv(r, g, p.g_m);
        off = (uint32_t)(sq - s_first) * qrow_b + (uint32_t)(r - sq * g) * qhead_b + (uint32_t)(ch * 16);
      }
      copy16_to_lds(rq, off, __builtin_amdgcn_readfirstlane(lds_q + j * 1024));
    }
  }
  // The valid key count (device-side seqused_k) is used only from here on,
  // so its load completes under the Q copies.
  __builtin_amdgcn_sched_barrier(0);
  const int nvalid = seqused_count(p, b, sq);
  blk.kbeg = SPLIT ? blk.z * p.kps : 0;
  if constexpr (CAUSAL) {
    blk.kend = SPLIT ? min(blk.kbeg + p.kps, kmax) : kmax;
    // the valid keys, up to the diagonal of the block's last row
    blk.kend = min(min(blk.kend, nvalid), udiv(min((blk.rb + 1) * ROWS, Mp) - 1, g, p.g_m) + (nvalid - sq.sq) + 1);
  } else {
    blk.kend = SPLIT ? min(blk.kbeg + p.kps, nvalid) : nvalid;
  }
  const int kbeg = blk.kbeg, kend = blk.kend;
  const int doff = CAUSAL ? nvalid - sq.sq : 0;  // causal: diagonal key offset (last query <-> last valid key)
  const int s_lo = udiv(min(row0, Mp - 1), g, p.g_m) + doff;

  typename G::E::v8 qf[QT][G::KC];
  int srow[QT];
  f32x4_t oacc[G::DT][QT];
#pragma unroll
  for (int i = 0; i < G::DT; ++i)
#pragma unroll
    for (int t = 0; t < QT; ++t) oacc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
  }
  const float c2 = p.scale_log2;

  // ---- this wave's K/V copies (see fwd_kernel: out-of-range keys read as 0)
  const uint32_t rstride_k = (uint32_t)(p.k_ss * 2), rstride_v = (uint32_t)(p.v_ss * 2);
  const u32x4_t rk = make_rsrc(p.k + view_off(b, sq.k0, hk, p.k_sb, p.k_ss, p.k_sh), (uint32_t)kend * rstride_k);
  const u32x4_t rv = make_rsrc(p.v + view_off(b, sq.k0, hk, p.v_sb, p.v_ss, p.v_sh), (uint32_t)kend * rstride_v);
  uint32_t voff_k[G::LPT_K], voff_v[G::LPT_V];
#pragma unroll
  for (int j = 0; j < G::LPT_K; ++j) {
    const int P = j * 64 + lane;
    const int row = P / (G::KSTR / 16), ch = P - row * (G::KSTR / 16);
    voff_k[j] = (ch < G::CPR) ? row * rstride_k + ch * 16 : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < G::LPT_V; ++j) {
    const int P = j * 64 + lane;
    const int row = P / (G::VSTR / 16), ch = P - row * (G::VSTR / 16);
    voff_v[j] = (ch < G::CPR) ? row * rstride_v + ch * 16 : kOutOfRange;
  }
  uint8_t* kbuf = smem + wave * WAVE_B;
  uint8_t* vbuf = RING ? kbuf : kbuf + (PIECES ? K_PIECES * 1024 : G::K_B);
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)kbuf);
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)vbuf);
  // A buffer is refilled only after this wave's reads of it have returned.
  auto issue_k = [&](int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const uint32_t toff = (uint32_t)kt * rstride_k;
#pragma unroll
    for (int j = 0; j < G::LPT_K; ++j) copy16_to_lds(rk, voff_k[j] + toff, lds_k + j * 1024);
  };
  auto issue_v = [&](int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const uint32_t toff = (uint32_t)kt * rstride_v;
#pragma unroll
    for (int j = 0; j < G::LPT_V; ++j) copy16_to_lds(rv, voff_v[j] + toff, lds_v + j * 1024);
  };

  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
  const int nown = ntiles > wave ? (ntiles - wave + KW - 1) / KW : 0;  // this wave's tiles

  // Piecewise refill: lane l of a piece copy fills quarter slot l % 4 of
  // key l / 4 of its 16 keys (with the quarter swizzles above).  `toff` is
  // the tile's byte offset in the buffer range, or kOutOfRange (past the
  // range: the copy writes zeros and reads no memory).
  const uint32_t pk_lane = (uint32_t)(lane >> 2) * rstride_k + ((uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  const uint32_t pv_lane = (uint32_t)(lane >> 2) * rstride_v + ((uint32_t)((lane & 3) ^ (((lane >> 4) & 1) << 1)) << 4);
  auto copy_k_piece = [&](uint32_t toff, int c, int mt) __attribute__((always_inline)) {
    copy16_to_lds(rk, pk_lane + (toff + (uint32_t)(16 * mt) * rstride_k + (uint32_t)(c * 64)),
                  lds_k + (c * G::MT + mt) * 1024);
  };
  auto copy_v_piece = [&](uint32_t toff, int e, int h) __attribute__((always_inline)) {
    copy16_to_lds(rv, pv_lane + (toff + (uint32_t)(16 * h) * rstride_v + (uint32_t)(e * 64)),
                  lds_v + (2 * e + h) * 1024);
  };

  // First K and V tiles after Q: waiting for all but the V copies then means
  // Q and K have landed, and the first QK^T overlaps the V copies.
  if (nown > 0) {
    if constexpr (PIECES) {
      const int kt0 = kbeg + wave * BN;
#pragma unroll
      for (int c = 0; c < G::KC; ++c)
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) copy_k_piece((uint32_t)kt0 * rstride_k, c, mt);
      // (the first V tile streams in during the first S^T)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(K_PIECES));  // this wave's Q copies landed
    } else {
      issue_k(kbeg + wave * BN);
      issue_v(kbeg + wave * BN);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(G::LPT_V));
    }
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  __syncthreads();  // every wave's part of the Q tile is in LDS

  // Q^T fragments from LDS: lane (col, grp) holds packed row row0 + 16t + col,
  // head-dim elements 32c + 8grp .. +7 (the row's rounding to 32 elements
  // holds zeros).
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int r = row0 + 16 * t + col;
    srow[t] = r < Mp ? udiv(r, g, p.g_m) + doff : -1;  // causal: the row's diagonal key
    // (ring: read from LDS at every S^T step instead, see read_q)
    if constexpr (!RING) {
#pragma unroll
      for (int c = 0; c < G::KC; ++c)
        qf[t][c] = G::E::cast(*reinterpret_cast<const u32x4_t*>(smem + Q_OFF + (16 * t + col) * QSTR + (4 * c + grp) * 16));
    }
  }

  uint32_t k_lane, v_lane;
  lane_bases<G>(lane, k_lane, v_lane);
  // Start the waves a quarter of a tile apart.  Every wave issues the 34
  // copies of its next K and V tiles in two bursts, and a burst stalls the
  // issuing wave while the compute unit's memory pipe (about 56 bytes per
  // clock) drains; waves that run in step all stall at once and then all
  // compute while the pipe idles.  Measured on the 968-key prefix shape:
  // 18.1 -> 16.0 us (4 x 64 clocks per wave index; 8 and 12 x 64 lose
  // part of the gain).
  for (int z = 0; z < wave; ++z) __builtin_amdgcn_s_sleep(4);
  if constexpr (PIECES) {
    // Reads of this lane: K fragment (key col of a piece, quarter grp
    // swizzled), V transpose read (key 4grp + r of a half, head-dim 4q of a
    // 16-element column u of the piece: quarter 2u + q/2, swizzled by the
    // key, which is 2(grp % 2) here).
    const uint32_t kr_lane = (uint32_t)(col * 4 + (grp ^ ((col >> 2) & 3))) * 16;
    const uint32_t vr_row = (uint32_t)((4 * grp + ((lane >> 2) & 3)) * 64 + ((lane & 3) >> 1) * 16 + (lane & 1) * 8);
    const uint8_t* kb = kbuf + kr_lane;
    const uint8_t* vb0 = vbuf + vr_row + 32 * (grp & 1);        // column u = 0
    const uint8_t* vb1 = vbuf + vr_row + 32 * (1 - (grp & 1));  // column u = 1
    // Copies retire in order, so a piece has landed once the copies issued
    // after it are all that is outstanding.  From the second tile on, before
    // a K piece of tile i is read those are at most: the rest of K(i), all of
    // V(i), and the K pieces of tile i+1 issued so far (PF steps behind the
    // reads): WK.  Likewise WV before a V read.  The first tile differs: its
    // V pieces are issued during its own S^T (step c: V(0) piece c, then
    // K(1) piece c), so that the S^T MFMAs overlap them; its counts follow
    // that order (k_wait, v_wait below, exact per read).  The last tile of a
    // wave issues no copies, so only the pieces of its own tile (and, in the
    // first tile, its V pieces) can follow a piece it reads.
    //
    // Ring scheme (two workgroups per compute unit, two waves per SIMD): a
    // wave has one 16 KiB buffer of KC slots of 2 KiB.  Slot c holds K
    // pieces (c, 0) and (c, 1) during S^T, then V piece c during O^T: in S^T
    // step c, once the reads of K slot c have returned, V(i) piece c is
    // issued into it, and in O^T, once both columns of V piece c have been
    // read, K(i+1) pieces (c, *) are.  Every tile (the first included, whose
    // K pieces the prologue issues) then sees the same order: before a K
    // read of tile i come only the later K(i) pieces and the V(i) pieces of
    // the earlier S^T steps; before a V read, the later V(i) pieces and the
    // K(i+1) pieces of the earlier O^T steps (none in a wave's last tile).
    // K steps whose fragments are read ahead of their MFMAs, and V fragments
    // read ahead.  The ring scheme has at most 256 registers per wave (two
    // waves per SIMD); it fits them, with no spills, because it reads the
    // Q^T fragments from LDS at every step (read_q) instead of holding all
    // 64 registers of them (holding them, it spilled around the first and
    // last tiles even with K one step and V four fragments ahead).
    constexpr int PF = 3;
    constexpr int PFV = 6;
    constexpr int WK = 2 * (G::KC - 1) + 2 * V_PIECES - 2 * PF;
    constexpr int WV = 2 * (V_PIECES - 1) + K_PIECES - PFV;
    static_assert(PFV % 2 == 0, "V reads run ahead by whole pieces");
    static_assert(G::MT == 2 && G::KVC == 1 && WK >= 0 && WV >= 0 && WK < 64 && WV < 64, "piece wait counts");
    static_assert(2 * V_PIECES == 2 * G::KC, "one V piece per K step of the first tile");
    // first tile: K(0) piece c' (prologue) is followed by the rest of K(0) and
    // 4 copies per S^T step issued before its read (at step c' - PF)
    auto k_wait = [](bool first, bool last, int c_read) constexpr -> int {
      const int ahead = c_read >= PF ? c_read - PF : 0;  // S^T steps whose copies precede the read
      if (RING) return 2 * (G::KC - 1 - c_read) + 2 * ahead;
      if (last) return 2 * (G::KC - 1 - c_read) + (first ? 2 * ahead : 2 * V_PIECES);
      return first ? 2 * (G::KC - 1 - c_read) + 4 * ahead : WK;
    };
    // first tile: V(0) piece e is followed by K(1) piece e, the later steps'
    // 4 copies, and the V(1) pieces issued before its read (after every
    // second O^T step)
    auto v_wait = [](bool first, bool last, int d_read) constexpr -> int {
      if (RING) return 2 * (V_PIECES - 1 - (d_read >> 1)) + (last || d_read < PFV ? 0 : 2 * ((d_read - PFV) >> 1));
      if (last) return 2 * (V_PIECES - 1 - (d_read >> 1));
      return first ? 2 + 4 * (V_PIECES - 1 - (d_read >> 1)) + 2 * (d_read >= PFV ? (d_read - PFV) >> 1 : 0) : WV;
    };
    // Ring: Q^T fragment of row 16t + col, head-dim step c (16-byte chunk
    // 4c + grp of the row, swizzled by the row).  The Q tile stays in LDS
    // until the merge, so the ring reads it at every S^T step instead of
    // holding all of Q^T in registers.
    auto read_q = [&](int c, int t) __attribute__((always_inline)) -> typename G::E::v8 {
      return G::E::cast(*reinterpret_cast<const u32x4_t*>(smem + Q_OFF + (16 * t + col) * QSTR + (((4 * c + grp) ^ col) * 16)));
    };
    auto read_k = [&](int c, int mt) __attribute__((always_inline)) -> typename G::E::v8 {
      return G::E::cast(*reinterpret_cast<const u32x4_t*>(kb + (c * G::MT + mt) * 1024));
    };
    auto read_v = [&](int dt) __attribute__((always_inline)) -> typename G::E::v8 {
      const uint8_t* vb = ((dt & 1) ? vb1 : vb0) + (dt >> 1) * 2048;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)vb);
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vb + 1024));
      const u32x4_t vw = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                          __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
      return G::E::cast(vw);
    };
    auto tile = [&](auto first_tag, auto last_tag, int i) __attribute__((always_inline)) {
      constexpr bool FIRST = decltype(first_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;  // no next tile: no copies
      const int kt = kbeg + (wave + i * KW) * BN;
      const uint32_t tk = (uint32_t)(kt + KW * BN) * rstride_k;  // the next tile of this wave
      const uint32_t tv = (uint32_t)(kt + KW * BN) * rstride_v;
      f32x4_t sacc[G::MT][QT];
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int t = 0; t < QT; ++t) sacc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      typename G::E::v8 kf[G::KC][G::MT];
      typename G::E::v8 qs[G::KC][QT];  // ring: Q^T fragments of the steps read ahead
      wait_vm(k_wait(FIRST, LAST, PF - 1));
#pragma unroll
      for (int c = 0; c < PF; ++c) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) kf[c][mt] = read_k(c, mt);
        if constexpr (RING) {
#pragma unroll
          for (int t = 0; t < QT; ++t) qs[c][t] = read_q(c, t);
        }
      }
#pragma unroll
      for (int c = 0; c < G::KC; ++c) {
        if (c + PF < G::KC) {
          wait_vm(k_wait(FIRST, LAST, c + PF));
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt) kf[c + PF][mt] = read_k(c + PF, mt);
          if constexpr (RING) {
#pragma unroll
            for (int t = 0; t < QT; ++t) qs[c + PF][t] = read_q(c + PF, t);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int t = 0; t < QT; ++t) sacc[mt][t] = G::E::mfma(kf[c][mt], RING ? qs[c][t] : qf[t][c], sacc[mt][t]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (RING) {
          // the reads of K slot c (and of its Q fragments) have returned:
          // V(i) piece c goes into it
          wait_lgkm((2 + QT) * (G::KC - 1 - c < PF ? G::KC - 1 - c : PF));
          copy_v_piece((uint32_t)kt * rstride_v, c, 0);
          copy_v_piece((uint32_t)kt * rstride_v, c, 1);
        } else if constexpr (FIRST) {
          copy_v_piece((uint32_t)kt * rstride_v, c, 0);  // the V buffer is not read before O^T
          copy_v_piece((uint32_t)kt * rstride_v, c, 1);
        }
        if constexpr (!LAST && !RING) {
          // the reads of step c have returned (fewer than 2 PF reads issued since)
          wait_lgkm(2 * (G::KC - 1 - c < PF ? G::KC - 1 - c : PF));
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt) copy_k_piece(tk, c, mt);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      uint32_t pk[G::KVC][QT][4];
      softmax_tile<G, QT, CAUSAL>(sacc, pk, m_run, l_run, oacc, srow, kt, kend, s_lo, c2, grp);
      __builtin_amdgcn_sched_barrier(0);
      typename G::E::v8 vf[G::DT];
      wait_vm(v_wait(FIRST, LAST, PFV - 1));
#pragma unroll
      for (int dt = 0; dt < PFV; ++dt) vf[dt] = read_v(dt);
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        if (dt + PFV < G::DT) {
          wait_vm(v_wait(FIRST, LAST, dt + PFV));
          vf[dt + PFV] = read_v(dt + PFV);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          const u32x4_t pw = {pk[0][t][0], pk[0][t][1], pk[0][t][2], pk[0][t][3]};
          oacc[dt][t] = G::E::mfma(vf[dt], G::E::cast(pw), oacc[dt][t]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!LAST && (dt & 1)) {
          // both columns of piece dt/2 have been read
          wait_lgkm(2 * (G::DT - 1 - dt < PFV ? G::DT - 1 - dt : PFV));
          if constexpr (RING) {
            copy_k_piece(tk, dt >> 1, 0);
            copy_k_piece(tk, dt >> 1, 1);
          } else {
            copy_v_piece(tv, dt >> 1, 0);
            copy_v_piece(tv, dt >> 1, 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (nown == 1) {
      tile(std::true_type{}, std::true_type{}, 0);
    } else if (nown > 1) {
      tile(std::true_type{}, std::false_type{}, 0);
      for (int i = 1; i < nown - 1; ++i) tile(std::false_type{}, std::false_type{}, i);
      tile(std::false_type{}, std::true_type{}, nown - 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the last copies have landed before the LDS is reused
  } else
  for (int i = 0; i < nown; ++i) {
    const int kt = kbeg + (wave + i * KW) * BN;
    const bool next = i + 1 < nown;
    if (i > 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(G::LPT_V));  // K(kt) landed; V(kt) may be in flight
    f32x4_t sacc[G::MT][QT];
    uint32_t pk[G::KVC][QT][4];
    qk_tile<G, QT>(sacc, qf, kbuf + k_lane, grp);
    if (next) issue_k(kt + KW * BN);  // the K buffer is free once the QK^T reads returned
    softmax_tile<G, QT, CAUSAL>(sacc, pk, m_run, l_run, oacc, srow, kt, kend, s_lo, c2, grp);
    __builtin_amdgcn_sched_barrier(0);
    if (next)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(G::LPT_K));  // V(kt) landed; the next K may be in flight
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    pv_tile<G, QT>(oacc, pk, kbuf + v_lane);  // v_lane already includes the K area
    if (next) issue_v(kt + KW * BN);
  }

  // ---- merge the KW partials through LDS.  Wave w stores its O (not yet
  // divided by l) and (m, l) per row; then TPR threads per row read every
  // wave's (m, l), form the weights 2^(m_w - M) / L (0 for a wave with no
  // keys) and sum the KW partials of their 16-byte chunks in wave order.
  // A wave's own buffer is idle once its last copies have landed (waited
  // for above) and its reads have returned (LDS operations of one wave run
  // in order), so it stores its O there without waiting for the others.
  auto o_chunk = [](int row, int c) constexpr -> int { return row * OSTR + (OSWZ ? (c ^ (row & 15)) : c) * 16; };
  float l_tot[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) l_tot[t] = group_sum(l_run[t]);
  float* mls = reinterpret_cast<float*>(smem + MLS_OFF);  // [row][wave] (m, l)
  // Wave stores of O rows 16t .. 16t+15 at row `orow` of the wave's buffer.
  auto store_o = [&](int t, int orow) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) {
      const int d = 16 * dt + 4 * grp;
      if (d < D) *reinterpret_cast<f32x4_t*>(kbuf + o_chunk(orow, d / 4)) = oacc[dt][t];
    }
  };
  auto store_ml = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int rl = 16 * t + col;
      if (grp == 0) *reinterpret_cast<u32x2_t*>(mls + 2 * (rl * KW + wave)) =
          u32x2_t{__float_as_uint(m_run[t]), __float_as_uint(l_tot[t])};
    }
  };
  // Merge of block rows rfirst .. rfirst+NR-1, whose O rows sit at rows
  // 0 .. NR-1 of every wave's buffer: TPR threads per row.
  auto merge_rows = [&](auto nr_tag, int rfirst) __attribute__((always_inline)) {
    constexpr int NR = decltype(nr_tag)::value;
    constexpr int TPR = KW * 64 / NR;  // threads per row
    static_assert(TPR * NR == KW * 64, "whole rows per workgroup pass");
    const int rl = rfirst + tid / TPR, c0 = tid - (tid / TPR) * TPR;
    const int orow = rl - rfirst;
    const int r = row0 + rl;
    if (r < Mp) {
      // Every LDS read of this thread is issued before any arithmetic: the
      // (m, l) pairs of the row and the KW partial chunks (a chain of dependent
      // read-then-multiply steps would keep only one or two reads in flight).
      constexpr int NJ = (G::CPR + TPR - 1) / TPR;
      f32x4_t part[NJ][KW][2];
      float mw[KW], fw[KW];
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        const u32x2_t ml = *reinterpret_cast<const u32x2_t*>(mls + 2 * (rl * KW + w));
        mw[w] = __uint_as_float(ml[0]);
        fw[w] = __uint_as_float(ml[1]);  // l of wave w
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int ch = min(c0 + TPR * j, G::CPR - 1);  // (a clamped chunk is read but not used)
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const uint8_t* src = smem + w * WAVE_B;
          part[j][w][0] = *reinterpret_cast<const f32x4_t*>(src + o_chunk(orow, 2 * ch));
          part[j][w][1] = *reinterpret_cast<const f32x4_t*>(src + o_chunk(orow, 2 * ch + 1));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < KW; ++w)
        if (fw[w] > 0.f) M = fmaxf(M, mw[w]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        const float e = fw[w] > 0.f ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.f;
        L += fw[w] * e;
        fw[w] = e;
      }
      const float inv = (L > 0.f) ? 1.0f / L : 0.f;
#pragma unroll
      for (int w = 0; w < KW; ++w) fw[w] *= inv;
      const int s = udiv(r, g, p.g_m), hh = r - s * g;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int ch = c0 + TPR * j;
        if (ch < G::CPR) {
          f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < KW; ++w) {
            a0 += fw[w] * part[j][w][0];
            a1 += fw[w] * part[j][w][1];
          }
          if constexpr (!SPLIT && OUTF == kOutNvfp4) {
            // chunks ch and ch ^ 1 form a block of 16; the other one is in the
            // neighbouring thread (tid ^ 1: same row, TPR even)
            float am = fmaxf(amax4(a0), amax4(a1));
            am = fmaxf(am, __shfl_xor(am, 1));
            float div;
            const uint32_t sc = nvfp4_scale(am, div);
            const size_t row = nvfp4_row(p, b, s, hk * g + hh);
            *reinterpret_cast<uint32_t*>(p.fp4_out + row * (D / 2) + 4 * ch) =
                nvfp4_pack4(a0, div) | (nvfp4_pack4(a1, div) << 16);
            if ((ch & 1) == 0) p.fp4_sf[row * (D / 16) + (ch >> 1)] = (uint8_t)sc;
          } else if constexpr (!SPLIT) {
            const u32x4_t o = {G::E::pack(a0[0], a0[1]), G::E::pack(a0[2], a0[3]), G::E::pack(a1[0], a1[1]),
                               G::E::pack(a1[2], a1[3])};
            *reinterpret_cast<u32x4_t*>(p.out + view_off(b, sq.q0 + s, hk * g + hh, p.o_sb, p.o_ss, p.o_sh) + 8 * ch) = o;
          } else {
            const size_t prow = (((size_t)bh * p.nrb + blk.rb) * p.zmax + blk.z) * ROWS + rl;
            float* po = p.ws_o + prow * D + 8 * ch;
            *reinterpret_cast<f32x4_t*>(po) = a0;
            *reinterpret_cast<f32x4_t*>(po + 4) = a1;
          }
        }
      }
      if (c0 == 0) {
        if constexpr (!SPLIT) {
          if (p.lse != nullptr)
            p.lse[sq.lse0 + (long long)(hk * g + hh) * p.lse_hs + s] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
        } else {
          const size_t prow = (((size_t)bh * p.nrb + blk.rb) * p.zmax + blk.z) * ROWS + rl;
          *reinterpret_cast<u32x2_t*>(p.ws_ml + 2 * prow) = u32x2_t{__float_as_uint(M), __float_as_uint(L)};
        }
      }
    }
  };
  if constexpr (RING) {
    // Two passes of 16 rows: the wave buffers hold 16 O rows each.
    store_o(0, col);
    __syncthreads();  // every wave is past its tiles and its Q reads: the Q area takes (m, l)
    store_ml();
    __syncthreads();
    merge_rows(std::integral_constant<int, 16>{}, 0);
#pragma unroll
    for (int t = 1; t < QT; ++t) {
      __syncthreads();  // the previous pass has read the buffers
      store_o(t, col);
      __syncthreads();
      merge_rows(std::integral_constant<int, 16>{}, 16 * t);
    }
  } else {
#pragma unroll
    for (int t = 0; t < QT; ++t) store_o(t, 16 * t + col);
    store_ml();
    __syncthreads();  // every wave's O and (m, l) are in LDS
    merge_rows(std::integral_constant<int, ROWS>{}, 0);
  }
}

// Merge of the split-KV partials of one packed row and 4 head-dim elements
// per thread (64-thread workgroups: the few rows of a split plan spread over
// more compute units), in split order (deterministic):
//   M = max_z m_z over non-empty splits, w_z = l_z 2^(m_z - M),
//   out = sum_z w_z Ohat_z / sum_z w_z,   lse = ln2 (M + log2 sum_z w_z).
// The running form below rescales as M grows, which is the same sum.
template <int D, int ROWS_WG, bool CAUSAL, int DTY, int OUTF>
__global__ void __launch_bounds__(64)
combine_kernel(const FwdParams p) {
  using E = Elem<DTY>;
  constexpr int CPR = D / 4;  // 4-element chunks per row: one per thread
  const int bh = blockIdx.y;  // (batch, kv head); x covers its row blocks
  const long long rem = (long long)blockIdx.x * 64 + threadIdx.x;
  if (rem >= (long long)p.nrb * ROWS_WG * CPR) return;
  const int rb = (int)(rem / (ROWS_WG * CPR));
  const int rl = (int)((rem / CPR) % ROWS_WG);
  const int ch = (int)(rem % CPR);
  const int r = rb * ROWS_WG + rl;
  const int g = p.g;
  const int b = udiv(bh, p.Hkv, p.hkv_m), hk = bh - b * p.Hkv;
  const Seq sq = seq_of(p, b);
  if (r >= sq.sq * g) return;  // past the end of this batch entry's queries
  int nz = p.zmax;
  if constexpr (CAUSAL) {
    nz = (causal_kmax_dev(p, rb, ROWS_WG) + p.kps - 1) / p.kps;
  }
  const size_t slot_base = ((size_t)bh * p.nrb + rb) * p.zmax;
  float M = -INFINITY, L = 0.f;
  f32x4_t a = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;  // splits whose loads are in flight together
  for (int z0 = 0; z0 < nz; z0 += U) {
    u32x2_t ml[U];
    f32x4_t o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int z = min(z0 + u, nz - 1);
      const size_t prow = (slot_base + z) * ROWS_WG + rl;
      ml[u] = *reinterpret_cast<const u32x2_t*>(p.ws_ml + 2 * prow);
      o[u] = *reinterpret_cast<const f32x4_t*>(p.ws_o + prow * D + 4 * ch);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float lz = __uint_as_float(ml[u][1]);
      if (z0 + u >= nz || !(lz > 0.f)) continue;
      const float mz = __uint_as_float(ml[u][0]);
      const float m_new = fmaxf(M, mz);
      const float alpha = __builtin_amdgcn_exp2f(M - m_new);  // 0 while M = -inf
      const float w = lz * __builtin_amdgcn_exp2f(mz - m_new);
      L = L * alpha + w;
      a = a * alpha + w * o[u];
      M = m_new;
    }
  }
  const int s = udiv(r, g, p.g_m), hh = r - s * g;
  const float inv = (L > 0.f) ? 1.0f / L : 0.f;
  if constexpr (OUTF == kOutNvfp4) {
    // a block of 16 is chunks 4j .. 4j+3, held by threads i with the same
    // i >> 2 (same row: D/4 is a multiple of 4)
    const f32x4_t x = a * inv;
    float am = amax4(x);
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    float div;
    const uint32_t sc = nvfp4_scale(am, div);
    const size_t row = nvfp4_row(p, b, s, hk * g + hh);
    *reinterpret_cast<uint16_t*>(p.fp4_out + row * (D / 2) + 2 * ch) = (uint16_t)nvfp4_pack4(x, div);
    if ((ch & 3) == 0) p.fp4_sf[row * (D / 16) + (ch >> 2)] = (uint8_t)sc;
  } else {
    const u32x2_t o = {E::pack(a[0] * inv, a[1] * inv), E::pack(a[2] * inv, a[3] * inv)};
    *reinterpret_cast<u32x2_t*>(p.out + view_off(b, sq.q0 + s, hk * g + hh, p.o_sb, p.o_ss, p.o_sh) + 4 * ch) = o;
  }
  if (ch == 0 && p.lse != nullptr) {
    const float lse = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
    p.lse[sq.lse0 + (long long)(hk * g + hh) * p.lse_hs + s] = lse;
  }
}

// ------------------------------------------------------------------ launch

template <int D, int QT, int NW, int BN, int NST, int KG, bool CAUSAL, bool SPLIT, int DTY, int OUTF = kOutElem>
static hipError_t launch_variant(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  using G = Geo<D, QT, NW, BN, DTY>;
  const int nrb = (p.Mp + G::ROWS_WG - 1) / G::ROWS_WG;
  dim3 grid;
  if (CAUSAL) {
    grid = dim3((unsigned)(nrb * (SPLIT ? std::max(p.zmax, 1) : 1)), p.B * p.Hkv, 1);
  } else {
    grid = dim3(nrb, p.B * p.Hkv, SPLIT ? plan.nsplit : 1);
  }
  hipLaunchKernelGGL((fwd_kernel<D, QT, NW, BN, NST, KG, CAUSAL, SPLIT, DTY, OUTF>), grid, dim3(NW * KG * 64), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !SPLIT) return e;
  const long long threads = (long long)nrb * G::ROWS_WG * (D / 4);  // per (batch, kv head)
  hipLaunchKernelGGL((combine_kernel<D, G::ROWS_WG, CAUSAL, DTY, OUTF>), dim3((unsigned)((threads + 63) / 64), p.B * p.Hkv),
                     dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int QT, int KW, int BN, int NST, bool CAUSAL, bool SPLIT, int DTY, int OUTF = kOutElem>
static hipError_t launch_ks_variant(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  constexpr int ROWS = 16 * QT;
  const int nrb = (p.Mp + ROWS - 1) / ROWS;
  dim3 grid;
  if (CAUSAL) {
    grid = dim3((unsigned)(nrb * (SPLIT ? std::max(p.zmax, 1) : 1)), p.B * p.Hkv, 1);
  } else {
    grid = dim3(nrb, p.B * p.Hkv, SPLIT ? plan.nsplit : 1);
  }
  hipLaunchKernelGGL((fwd_ks_kernel<D, QT, KW, BN, NST, CAUSAL, SPLIT, DTY, OUTF>), grid, dim3(KW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !SPLIT) return e;
  const long long threads = (long long)nrb * ROWS * (D / 4);  // per (batch, kv head)
  hipLaunchKernelGGL((combine_kernel<D, ROWS, CAUSAL, DTY, OUTF>), dim3((unsigned)((threads + 63) / 64), p.B * p.Hkv), dim3(64),
                     0, stream, p);
  return hipGetLastError();
}

// The compiled variants.  Row-split (fwd_kernel) entries: element type, head
// dim, rows per wave / 16, waves per key group, key groups, keys per tile,
// K/V stages in LDS (two: one tile computed while the next loads; three or
// more: the software-pipelined loop).  With two key groups the workgroup
// has twice the waves on the same rows, each group taking every other key
// tile, and the two partials are merged in LDS.  Key-split (fwd_ks_kernel)
// entries: element type, head dim, rows per wave / 16, waves (all on the
// same rows), keys per tile, buffer scheme (1: whole-tile buffers, 2:
// piecewise refill).  Every variant is built with and without causal
// masking and with and without the split-KV partial output.  fp16 has the
// variants the default plan uses.
#define FA_VARIANTS(X)           \
  X(kBf16, 64, 1, 4, 1, 64, 2)   \
  X(kBf16, 64, 1, 4, 1, 128, 2)  \
  X(kBf16, 64, 2, 2, 1, 64, 2)   \
  X(kBf16, 64, 2, 4, 1, 64, 2)   \
  X(kBf16, 64, 1, 4, 1, 64, 3)   \
  X(kBf16, 64, 1, 4, 2, 64, 2)   \
  X(kBf16, 64, 1, 2, 2, 64, 2)   \
  X(kBf16, 72, 1, 4, 1, 64, 2)   \
  X(kBf16, 72, 1, 4, 1, 128, 2)  \
  X(kBf16, 72, 1, 4, 1, 64, 3)   \
  X(kBf16, 72, 1, 4, 1, 64, 4)   \
  X(kBf16, 72, 2, 2, 1, 64, 2)   \
  X(kBf16, 72, 2, 2, 1, 64, 3)   \
  X(kBf16, 72, 2, 4, 1, 64, 2)   \
  X(kBf16, 72, 1, 4, 2, 64, 2)   \
  X(kBf16, 72, 1, 2, 2, 64, 2)   \
  X(kBf16, 256, 1, 4, 1, 32, 2)  \
  X(kBf16, 256, 1, 4, 1, 32, 4)  \
  X(kBf16, 256, 1, 4, 1, 64, 2)  \
  X(kBf16, 256, 2, 4, 1, 32, 2)  \
  X(kBf16, 256, 2, 4, 1, 32, 4)  \
  X(kBf16, 256, 2, 4, 1, 64, 2)  \
  X(kF16, 64, 1, 4, 1, 64, 2)    \
  X(kF16, 64, 1, 4, 1, 128, 2)   \
  X(kF16, 72, 1, 4, 1, 64, 2)    \
  X(kF16, 72, 1, 4, 1, 128, 2)   \
  X(kF16, 64, 1, 4, 2, 64, 2)    \
  X(kF16, 64, 1, 2, 2, 64, 2)    \
  X(kF16, 72, 1, 4, 2, 64, 2)    \
  X(kF16, 72, 1, 2, 2, 64, 2)    \
  X(kF16, 64, 2, 4, 1, 64, 2)    \
  X(kF16, 72, 2, 4, 1, 64, 2)    \
  X(kF16, 256, 2, 4, 1, 32, 2)   \
  X(kF16, 256, 1, 4, 1, 64, 2)

#define FA_KS_VARIANTS(X)     \
  X(kBf16, 64, 2, 4, 64, 1)   \
  X(kBf16, 72, 2, 4, 64, 1)   \
  X(kBf16, 256, 2, 4, 32, 1)  \
  X(kBf16, 256, 1, 4, 32, 1)  \
  X(kBf16, 256, 2, 2, 32, 1)  \
  X(kBf16, 256, 2, 4, 32, 2)  \
  X(kBf16, 256, 2, 4, 32, 3)  \
  X(kBf16, 256, 1, 4, 32, 2)  \
  X(kF16, 256, 2, 4, 32, 2)   \
  X(kF16, 256, 2, 4, 32, 3)   \
  X(kF16, 256, 1, 4, 32, 2)

// (nw, kw) of a plan: kw == 1, waves on different rows; kw == nw, every wave
// on the same rows (key-split kernel);
// otherwise kw key groups of nw / kw waves each (row-split kernel).
bool variant_exists(int D, int qt, int nw, int kw, int bn, int nst, int dtype) {
  if (kw < 1 || nw < kw || nw % kw != 0) return false;
  if (kw == 1 || kw < nw) {
    const int n = nw / kw;
#define FA_MATCH(t_, d_, q_, n_, g_, b_, s_) \
  if (dtype == t_ && D == d_ && qt == q_ && n == n_ && kw == g_ && bn == b_ && nst == s_) return true;
    FA_VARIANTS(FA_MATCH)
#undef FA_MATCH
    return false;
  }
#define FA_KS_MATCH(t_, d_, q_, k_, b_, s_) \
  if (dtype == t_ && D == d_ && qt == q_ && kw == k_ && bn == b_ && nst == s_) return true;
  FA_KS_VARIANTS(FA_KS_MATCH)
#undef FA_KS_MATCH
  return false;
}

// NVFP4 output: built for the default bf16 plans of the head dims whose rows
// split into whole blocks of 16 (row-split at 64, key-split at 256).
bool nvfp4_variant_exists(const LaunchPlan& l) {
  return l.dtype == kBf16 && ((l.D == 64 && l.qt == 1 && l.nw == 4 && l.kw == 1 && (l.bn == 64 || l.bn == 128) &&
                               l.nst == 2) ||
                              (l.D == 64 && l.qt == 1 && (l.nw == 4 || l.nw == 8) && l.kw == 2 && l.bn == 64 &&
                               l.nst == 2) ||
                              (l.D == 64 && l.qt == 2 && l.nw == 4 && l.kw == 1 && l.bn == 64 && l.nst == 2) ||
                              (l.D == 256 && l.qt == 2 && l.nw == 4 && l.kw == 1 && l.bn == 32 && l.nst == 2) ||
                              (l.D == 256 && l.qt == 1 && l.nw == 4 && l.kw == 1 && l.bn == 64 && l.nst == 2) ||
                              (l.D == 256 && (l.qt == 1 || l.qt == 2) && l.nw == 4 && l.kw == 4 && l.bn == 32 &&
                               l.nst == 2) ||
                              (l.D == 256 && l.qt == 2 && l.nw == 4 && l.kw == 4 && l.bn == 32 && l.nst == 3));
}

template <bool CAUSAL, bool SPLIT>
static hipError_t launch_nvfp4(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  if (plan.D == 256 && plan.kw == 1)
    return plan.qt == 2 ? launch_variant<256, 2, 4, 32, 2, 1, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream)
                        : launch_variant<256, 1, 4, 64, 2, 1, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
  if (plan.D == 64 && plan.qt == 2)
    return launch_variant<64, 2, 4, 64, 2, 1, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
  if (plan.D == 64 && plan.kw == 2)
    return plan.nw == 8 ? launch_variant<64, 1, 4, 64, 2, 2, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream)
                        : launch_variant<64, 1, 2, 64, 2, 2, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
  if (plan.D == 64)
    return plan.bn == 128 ? launch_variant<64, 1, 4, 128, 2, 1, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream)
                          : launch_variant<64, 1, 4, 64, 2, 1, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
  if (plan.nst == 3) return launch_ks_variant<256, 2, 4, 32, 3, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
  return plan.qt == 1 ? launch_ks_variant<256, 1, 4, 32, 2, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream)
                      : launch_ks_variant<256, 2, 4, 32, 2, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
}

hipError_t launch_fwd(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  if (plan.outf == kOutNvfp4) {
    if (!nvfp4_variant_exists(plan)) return hipErrorInvalidValue;
    if (plan.causal)
      return plan.split ? launch_nvfp4<true, true>(p, plan, stream) : launch_nvfp4<true, false>(p, plan, stream);
    return plan.split ? launch_nvfp4<false, true>(p, plan, stream) : launch_nvfp4<false, false>(p, plan, stream);
  }
  if (plan.kw > 1 && plan.kw == plan.nw) {
#define FA_KS_DISPATCH(t_, d_, q_, k_, b_, s_)                                                          \
  if (plan.dtype == t_ && plan.D == d_ && plan.qt == q_ && plan.kw == k_ && plan.bn == b_ && plan.nst == s_) { \
    if (plan.causal)                                                                                    \
      return plan.split ? launch_ks_variant<d_, q_, k_, b_, s_, true, true, t_>(p, plan, stream)        \
                        : launch_ks_variant<d_, q_, k_, b_, s_, true, false, t_>(p, plan, stream);      \
    return plan.split ? launch_ks_variant<d_, q_, k_, b_, s_, false, true, t_>(p, plan, stream)         \
                      : launch_ks_variant<d_, q_, k_, b_, s_, false, false, t_>(p, plan, stream);       \
  }
    FA_KS_VARIANTS(FA_KS_DISPATCH)
#undef FA_KS_DISPATCH
    return hipErrorInvalidValue;
  }
  if (plan.kw < 1 || plan.nw % plan.kw != 0) return hipErrorInvalidValue;
  const int n = plan.nw / plan.kw;
#define FA_DISPATCH(t_, d_, q_, n_, g_, b_, s_)                                                        \
  if (plan.dtype == t_ && plan.D == d_ && plan.qt == q_ && n == n_ && plan.kw == g_ && plan.bn == b_ && \
      plan.nst == s_) {                                                                                \
    if (plan.causal)                                                                                   \
      return plan.split ? launch_variant<d_, q_, n_, b_, s_, g_, true, true, t_>(p, plan, stream)      \
                        : launch_variant<d_, q_, n_, b_, s_, g_, true, false, t_>(p, plan, stream);    \
    return plan.split ? launch_variant<d_, q_, n_, b_, s_, g_, false, true, t_>(p, plan, stream)       \
                      : launch_variant<d_, q_, n_, b_, s_, g_, false, false, t_>(p, plan, stream);     \
  }
  FA_VARIANTS(FA_DISPATCH)
#undef FA_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace fa
