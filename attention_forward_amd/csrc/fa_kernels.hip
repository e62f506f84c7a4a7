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

#include "fa_launch.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

static constexpr float kLn2 = 0.6931471805599453f;
static constexpr float kRescaleThreshold = 8.0f;  // log2 units: rescale when the max grows by > 2^8
constexpr int kRawBufferFlags = 0x00020000;       // dword 3 of a raw (untyped) buffer resource on gfx9
constexpr uint32_t kOutOfRange = 0x80000000u;     // a buffer offset past any range: reads as zero

// s_waitcnt immediate with vmcnt = n and expcnt / lgkmcnt left at their
// maxima (vmcnt is split over bits 3:0 and 15:14).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate with lgkmcnt = 0 (every LDS access of this wave has
// completed) and vmcnt / expcnt left at their maxima.
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  f16x2_t r = {(_Float16)lo, (_Float16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// Element type of q, k, v and out: the MFMA that consumes eight of them per
// lane, and the rounding of P and of the output.
template <int DTY>
struct Elem;
template <>
struct Elem<kBf16> {
  typedef bf16x8_t v8;
  static __device__ __forceinline__ v8 cast(u32x4_t x) { return __builtin_bit_cast(v8, x); }
  static __device__ __forceinline__ f32x4_t mfma(v8 a, v8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) { return pack_bf16x2(lo, hi); }
};
template <>
struct Elem<kF16> {
  typedef f16x8_t v8;
  static __device__ __forceinline__ v8 cast(u32x4_t x) { return __builtin_bit_cast(v8, x); }
  static __device__ __forceinline__ f32x4_t mfma(v8 a, v8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) { return pack_f16x2(lo, hi); }
};

// x combined over lanes l, l^16, l^32, l^48 (the four 16-lane rows that hold
// one accumulator column).  permlane32_swap(x, x) gives {x[l & 31], x[l | 32]}
// per lane, permlane16_swap(x, x) gives {x[l & ~16], x[l | 16]}.
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------- NVFP4 output
// The attention output quantised for the output projection: per (token,
// head) row, blocks of 16 head-dim elements; a block's scale is amax/6 in
// fp32 rounded to UE4M3 (4-bit exponent bias 7, 3-bit mantissa, subnormals
// m/8 * 2^-6, largest finite 448; nearest, ties to the even code,
// saturating), and each element x / (decoded scale) in fp32 rounded to E2M1
// (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; nearest, ties to the even code,
// saturating at 6; sign bit when x < 0), decided without the division
// (e2m1_cuts).  A block whose scale rounds to zero
// gets zero codes.  Two elements per byte, the even one in the low nibble.

__device__ __forceinline__ uint32_t ue4m3_code(float v) {
  if (!(v > 0.f)) return 0u;
  if (v >= 448.f) return 0x7Eu;
  const int e = (int)((__float_as_uint(v) >> 23) & 0xFF) - 127;  // floor(log2 v) for normal floats
  if (e < -6) {
    const float q = __builtin_rintf(v * 512.f);  // multiples of 2^-9, ties to even
    return q >= 8.f ? 0x08u : (uint32_t)q;
  }
  float q = __builtin_rintf(__builtin_ldexpf(v, -e) * 8.f);  // mantissa in eighths: 8 .. 16
  int ee = e;
  if (q >= 16.f) {
    q = 8.f;
    ee += 1;
  }
  return ((uint32_t)(ee + 7) << 3) | ((uint32_t)q - 8u);
}

__device__ __forceinline__ float ue4m3_float(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e == 0 ? (float)m * 0.001953125f : __builtin_ldexpf(1.f + (float)m * 0.125f, (int)e - 7);
}

// E2M1 decision points of a block: the midpoints between neighbouring
// magnitudes (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) times the decoded scale.
// Each product is exact (a short dyadic times a scale of at most 4
// significant bits), and an fp32 x that is not exactly such a product is
// more than half an ulp of the midpoint away from it after division, so
// comparing |x| with the products decides exactly as rounding the fp32
// quotient x / scale and comparing that with the midpoints.
struct E2m1Cuts {
  float c[7];
};

__device__ __forceinline__ E2m1Cuts e2m1_cuts(float scale) {
  return E2m1Cuts{{0.25f * scale, 0.75f * scale, 1.25f * scale, 1.75f * scale, 2.5f * scale, 3.5f * scale,
                   5.f * scale}};
}

// E2M1 code: the magnitude code counts the decision points passed (strict at
// a midpoint whose lower neighbour has the even code).
__device__ __forceinline__ uint32_t e2m1_code(float x, const E2m1Cuts& k) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > k.c[0]) + (uint32_t)(a >= k.c[1]) + (uint32_t)(a > k.c[2]) +
                     (uint32_t)(a >= k.c[3]) + (uint32_t)(a > k.c[4]) + (uint32_t)(a >= k.c[5]) + (uint32_t)(a > k.c[6]);
  return c | (x < 0.f ? 8u : 0u);
}

// Scale code of a block from its amax, and the decoded scale its elements
// use (0: the block is coded as zeros).
__device__ __forceinline__ uint32_t nvfp4_scale(float amax, float& scale) {
  const uint32_t sc = ue4m3_code(amax / 6.f);
  scale = ue4m3_float(sc);
  return sc;
}

// Four elements (x0..x3) of a block -> four nibbles (16 bits, x0 lowest).
__device__ __forceinline__ uint32_t nvfp4_pack4(f32x4_t x, float scale) {
  if (!(scale > 0.f)) return 0u;
  const E2m1Cuts k = e2m1_cuts(scale);
  return e2m1_code(x[0], k) | (e2m1_code(x[1], k) << 4) | (e2m1_code(x[2], k) << 8) | (e2m1_code(x[3], k) << 12);
}

__device__ __forceinline__ float amax4(f32x4_t x) {
  return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
}

// Byte offset of (batch b, position s, head h)'s row in the NVFP4 output
// (rows of D/2 code bytes; the scales use rows of D/16 bytes).
__device__ __forceinline__ size_t nvfp4_row(const FwdParams& p, int b, int s, int h) {
  return ((size_t)b * p.Sq + s) * p.Hq + h;
}

// One 16-byte copy per lane from a buffer to LDS (buffer_load_dwordx4 with
// the LDS bit): lane i of the wave writes LDS bytes [lds + 16 i, +16) with
// the 16 bytes at buffer offset voff, or zeros when that offset is past the
// buffer's range.  Inline asm so that the compiler adds no waits for
// it in front of later LDS reads: the main loop waits for these copies
// itself (s_waitcnt vmcnt and a barrier before a stage is read).  The
// instruction has no register result; M0 carries the wave-uniform LDS
// address and is used by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(u32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// Raw buffer resource (stride 0, byte range `bytes`) for a wave-uniform base
// address, built in scalar registers.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kRawBufferFlags};
}
#pragma clang diagnostic pop

constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
// Smallest LDS row stride >= bytes that is an odd multiple of 16 bytes, or
// 32 modulo 128 bytes (V rows; see Geo).
constexpr int odd16_stride(int bytes) { return (bytes % 32 == 16) ? bytes : odd16_stride(bytes + 16); }
constexpr int mod128_stride(int bytes) { return (bytes % 128 == 32) ? bytes : mod128_stride(bytes + 16); }

// Compile-time geometry of one kernel variant.
template <int D, int QT, int NW, int BN, int DTY = kBf16>
struct Geo {
  using E = Elem<DTY>;                           // element type of q, k, v, out
  static constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  static constexpr int ROWB = D * 2;             // bytes per K/V row
  // LDS row strides, chosen by measurement on gfx950.  A K row holds the
  // head dim rounded up to the 32-element MFMA step (the rounding is filled
  // with zeros by the tile copies, so the last step of S^T = K Q^T needs no
  // per-lane guard) plus padding; a V row is at least as long as the
  // fragment reads of the last head-dim tile (the transpose reads take 32
  // bytes from each of 4 rows).  In isolation, 16 rows read at one column
  // with 16-byte loads run at the rate of contiguous reads when the K stride
  // is 32 modulo 64 bytes (17% slower at 16 modulo 64), and the transpose
  // reads are 10% faster when the V stride is an odd multiple of 16 bytes.
  // In the kernels the two interact: with both, the 256-wide key-split
  // kernel is 4% slower.  Whole-kernel timings pick 32 bytes of K padding
  // with V rows 32 modulo 128 for head dims up to 128 (the 72-wide workload
  // 4% faster), and 16 bytes with odd-multiple V rows above (1-2% faster).
  static constexpr bool WIDE = D > 128;
  static constexpr int KSTR = round_up(D, 32) * 2 + (WIDE ? 16 : 32);
  static constexpr int VSTR = WIDE ? odd16_stride(round_up(D, 16) * 2) : mod128_stride(round_up(D, 16) * 2);
  static constexpr int NT = NW * 64;             // threads
  static constexpr int K_SLOTS = round_up(BN * (KSTR / 16), 64);  // 16-byte slots per K tile
  static constexpr int V_SLOTS = round_up(BN * (VSTR / 16), 64);
  static constexpr int LPT_K = (K_SLOTS + NT - 1) / NT;  // copies per thread per K tile
  static constexpr int LPT_V = (V_SLOTS + NT - 1) / NT;
  static constexpr int LPT = LPT_K + LPT_V;
  static constexpr bool TRASH = (K_SLOTS % NT) != 0 || (V_SLOTS % NT) != 0;
  static constexpr int K_B = K_SLOTS * 16;
  static constexpr int STAGE_B = K_B + V_SLOTS * 16;  // K tile then V tile
  static constexpr int KC = (D + 31) / 32;       // K steps of S^T = K Q^T
  static constexpr int DT = (D + 15) / 16;       // 16-row tiles of O^T
  static constexpr int MT = BN / 16;             // 16-key tiles of S^T
  static constexpr int KVC = BN / 32;            // 32-key K steps of O^T
  static constexpr int ROWS_WG = NW * 16 * QT;
  static_assert(D % 8 == 0, "head dim must be a multiple of 8");
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  static_assert(DT * 16 * 2 <= VSTR, "V fragment reads stay inside a padded row");
};

// ---------------------------------------------------------------- tile phases
// The three phases of one K/V tile for a wave that owns 16*QT packed rows.
// G is the kernel geometry (head dim, key tile, LDS strides).  `kb` and
// `vb` are this lane's read bases in the K and V tiles (see lane_bases).

// Per-lane LDS read bases inside a stage: K fragment (row col of a 16-key
// tile, chunk grp of a 32-element step), V transpose read (row 4grp + r,
// head-dim 4q).
template <class G>
__device__ __forceinline__ void lane_bases(int lane, uint32_t& k_lane, uint32_t& v_lane) {
  const int col = lane & 15, grp = lane >> 4, vr = lane >> 2 & 3, vq = lane & 3;
  k_lane = col * G::KSTR + grp * 16;
  v_lane = G::K_B + (4 * grp + vr) * G::VSTR + vq * 8;
}

// S^T = K * Q^T for one tile: lane (col, grp) gets query col, keys
// 16mt + 4grp + r.  Fragment loads run a few steps ahead of the MFMAs that
// use them; the scheduling barriers keep that order so LDS latency overlaps
// MFMA work.
template <class G, int QT>
__device__ __forceinline__ void qk_tile(f32x4_t (&sacc)[G::MT][QT], const typename G::E::v8 (&qf)[QT][G::KC],
                                        const uint8_t* kb, int grp) {
  auto load_k = [&](int c, int mt) __attribute__((always_inline)) -> typename G::E::v8 {
    return G::E::cast(*reinterpret_cast<const u32x4_t*>(kb + mt * 16 * G::KSTR + c * 64));
  };
  constexpr int PFK = G::KC < 3 ? G::KC : 3;
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int t = 0; t < QT; ++t) sacc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  typename G::E::v8 kf[G::KC][G::MT];
#pragma unroll
  for (int c = 0; c < PFK; ++c)
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) kf[c][mt] = load_k(c, mt);
#pragma unroll
  for (int c = 0; c < G::KC; ++c) {
    if (c + PFK < G::KC) {
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) kf[c + PFK][mt] = load_k(c + PFK, mt);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int t = 0; t < QT; ++t)
        sacc[mt][t] = G::E::mfma(kf[c][mt], qf[t][c], sacc[mt][t]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// V^T fragment for 32-key step kc and head-dim tile dt.  Lane 16grp+4r+q of
// read h points at V row 32kc + 16h + 4grp + r, head-dim 16dt + 4q..+3; the
// transpose read hands lane (col, grp) the four keys of that group at
// head-dim 16dt + col, i.e. the slots P^T holds in elements 4h .. 4h+3.
// Past the head dim (D = 72, dt = 4) the reads land in the row padding.
template <class G>
__device__ __forceinline__ typename G::E::v8 load_v(const uint8_t* vb, int kc, int dt) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vb + (32 * kc) * G::VSTR + dt * 32));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vb + (32 * kc + 16) * G::VSTR + dt * 32));
  const u32x4_t vw = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                      __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
  return G::E::cast(vw);
}

// Online softmax of one tile on the raw scores (scale > 0, so the max
// commutes with it): p = exp2(s * scale*log2e - m) in one fma + exp.  Keys
// at or past kend, and for causal keys past the row's position, get p = 0.
// Updates m_run / l_run, rescales O lazily, and packs P^T to bf16.
// The mask is needed only where the tile crosses the end of the key range or
// (causal) the diagonal of the wave's first row.  It is applied in a real
// branch (the scheduling barrier inside cannot be speculated), so full tiles
// run no per-element compare and select.
template <class G, int QT, bool CAUSAL>
__device__ __forceinline__ void softmax_tile(f32x4_t (&sacc)[G::MT][QT], uint32_t (&pk)[G::KVC][QT][4],
                                             float (&m_run)[QT], float (&l_run)[QT],
                                             f32x4_t (&oacc)[G::DT][QT], const int (&srow)[QT], int kt, int kend,
                                             int s_lo, float c2, int grp) {
  constexpr int BN = G::MT * 16;
  if ((kt + BN > kend) || (CAUSAL && kt + BN - 1 > s_lo)) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      // Element (mt, r) of this lane is key kt + 4grp + 16mt + r; it is kept
      // while 16mt + r is below the lane's limit.
      int lim = kend - kt - 4 * grp;
      if constexpr (CAUSAL) lim = min(lim, srow[t] + 1 - kt - 4 * grp);
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[mt][t][r] = (16 * mt + r < lim) ? sacc[mt][t][r] : -INFINITY;
    }
  }
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[mt][t][r]);
    mx = group_max(mx) * c2;
    const float m_new = fmaxf(m_run[t], mx);
    // The branch is taken when any row of the wave moves; each row then
    // rescales by its own factor (1 for a row whose max stayed, including a
    // row that has attended no key yet, whose max is still -inf).
    const bool moved = m_new > m_run[t] + kRescaleThreshold;
    if (__ballot(moved) != 0) {
      const float alpha = moved ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;  // 0 when m_run = -inf
      m_run[t] = moved ? m_new : m_run[t];
      l_run[t] *= alpha;
#pragma unroll
      for (int i = 0; i < G::DT; ++i) oacc[i][t] *= alpha;
    }
    const float m_neg = (m_run[t] == -INFINITY) ? 0.f : -m_run[t];
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][t][r], c2, m_neg));
        sacc[mt][t][r] = pv;
        lsum += pv;
      }
    l_run[t] += lsum;
#pragma unroll
    for (int kc = 0; kc < G::KVC; ++kc) {
      pk[kc][t][0] = G::E::pack(sacc[2 * kc][t][0], sacc[2 * kc][t][1]);
      pk[kc][t][1] = G::E::pack(sacc[2 * kc][t][2], sacc[2 * kc][t][3]);
      pk[kc][t][2] = G::E::pack(sacc[2 * kc + 1][t][0], sacc[2 * kc + 1][t][1]);
      pk[kc][t][3] = G::E::pack(sacc[2 * kc + 1][t][2], sacc[2 * kc + 1][t][3]);
    }
  }
}

// O^T += V^T * P^T for one tile: lane (col, grp) gets query col, head-dim
// 16dt + 4grp + r.
template <class G, int QT>
__device__ __forceinline__ void pv_tile(f32x4_t (&oacc)[G::DT][QT], const uint32_t (&pk)[G::KVC][QT][4],
                                        const uint8_t* vb) {
  constexpr int NV = G::KVC * G::DT;
  constexpr int PFA = G::WIDE ? 6 : 4;  // reads in flight: measured per head-dim class
  constexpr int PFV = NV < PFA ? NV : PFA;
  typename G::E::v8 vf[NV];
#pragma unroll
  for (int i = 0; i < PFV; ++i) vf[i] = load_v<G>(vb, i / G::DT, i % G::DT);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int kc = i / G::DT, dt = i % G::DT;
    if (i + PFV < NV) vf[i + PFV] = load_v<G>(vb, (i + PFV) / G::DT, (i + PFV) % G::DT);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const u32x4_t pw = {pk[kc][t][0], pk[kc][t][1], pk[kc][t][2], pk[kc][t][3]};
      oacc[dt][t] = G::E::mfma(vf[i], G::E::cast(pw), oacc[dt][t]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroups are dispatched to the eight XCDs round-robin in linear block
// order, and each XCD has its own L2.  For a non-causal single-pass grid
// whose (batch, kv head) count is a multiple of 8, block n is given to
// (batch*kv head, row block) such that every row block of one (batch, kv
// head) lands on the same XCD and its K/V is fetched into one L2 only.
// The grid sizes come from the launch parameters (nrb row blocks by B*Hkv),
// not from the dispatch packet, which would take two more dependent scalar
// loads before the first tile copy.
// n / d for 0 <= n < 2^31 and d >= 1, given m = floor((2^32 - 1) / d): the
// high half of n*m is the quotient or one less (m > (2^32 - 1) / d - 1 and
// n < 2^31 keep the error of n*m / 2^32 below one), so one correction step
// makes it exact.  Scalar multiplies only, where the compiler's division
// would go through a vector reciprocal and back.
__device__ __forceinline__ int udiv(int n, int d, uint32_t m) {
  const uint32_t q = __umulhi((uint32_t)n, m);
  return (int)(q + ((uint32_t)n - q * (uint32_t)d >= (uint32_t)d ? 1u : 0u));
}

__device__ __forceinline__ void xcd_block(const FwdParams& p, int& bh, int& rb) {
  bh = blockIdx.y;
  rb = blockIdx.x;
  const int nbh = p.B * p.Hkv;
  if ((nbh & 7) == 0) {
    const int n = blockIdx.x + p.nrb * blockIdx.y;  // dispatch order
    const int slot = n >> 3, grp = udiv(slot, p.nrb, p.nrb_m);
    bh = (n & 7) + 8 * grp;
    rb = slot - grp * p.nrb;
  }
}

// Loads the launch parameters the prologue needs at kernel entry, together:
// the compiler would otherwise fetch the strides only after the first
// branch, one more scalar-memory round trip before the first tile copy.
__device__ __forceinline__ void pin_params(const FwdParams& p) {
  asm volatile("" ::"s"(p.q_sb), "s"(p.q_ss), "s"(p.q_sh), "s"(p.k_sb), "s"(p.k_ss), "s"(p.k_sh), "s"(p.v_sb),
               "s"(p.v_ss), "s"(p.v_sh), "s"(p.o_ss), "s"(p.o_sh), "s"(p.o_sb));
  asm volatile("" ::"s"(p.nrb), "s"(p.nrb_m), "s"(p.hkv_m), "s"(p.kps), "s"(p.coff), "s"(p.zmax), "s"(p.Mp),
               "s"(p.lse_hs), "s"(p.lse_bs), "s"(p.total_q), "s"(p.total_k));
}

// ---- straight-line tile phases for the software-pipelined loop
// S^T = K * Q^T with every K fragment loaded up front and no scheduling
// barriers, so the compiler may interleave these MFMAs with other work.
template <class G, int QT>
__device__ __forceinline__ void qk_flat(f32x4_t (&sacc)[G::MT][QT], const typename G::E::v8 (&qf)[QT][G::KC],
                                        const uint8_t* kb) {
  typename G::E::v8 kf[G::KC][G::MT];
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
      kf[c][mt] = G::E::cast(*reinterpret_cast<const u32x4_t*>(kb + mt * 16 * G::KSTR + c * 64));
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int t = 0; t < QT; ++t) sacc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int t = 0; t < QT; ++t)
        sacc[mt][t] = G::E::mfma(kf[c][mt], qf[t][c], sacc[mt][t]);
}

// The mask of softmax_tile on its own (a real branch, taken only by tiles
// that cross the end of the key range or a causal diagonal).
template <class G, int QT, bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x4_t (&sacc)[G::MT][QT], const int (&srow)[QT], int kt, int kend,
                                          int s_lo, int grp) {
  constexpr int BN = G::MT * 16;
  if ((kt + BN > kend) || (CAUSAL && kt + BN - 1 > s_lo)) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      int lim = kend - kt - 4 * grp;
      if constexpr (CAUSAL) lim = min(lim, srow[t] + 1 - kt - 4 * grp);
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[mt][t][r] = (16 * mt + r < lim) ? sacc[mt][t][r] : -INFINITY;
    }
  }
}

// One step of the software-pipelined loop: S^T of the next tile (K fragments
// at `kn`) into s_nxt, overlapped with the softmax of the current tile
// (s_cur, already masked) into pk.  The softmax has no branches: the lazy
// rescale is decided per row and every row multiplies O and l by its factor
// (1 when its max did not move).  The work is laid out in three phases
// separated by scheduling barriers, each pairing a third of the S^T MFMAs
// with independent VALU work: the row max, then the reductions and the
// rescale, then the exponentials, sums and bf16 packing.  The MFMAs run on
// the matrix core while the wave issues the VALU instructions.
template <class G, int QT>
__device__ __forceinline__ void pipe_tile(f32x4_t (&s_nxt)[G::MT][QT], f32x4_t (&s_cur)[G::MT][QT],
                                          const typename G::E::v8 (&qf)[QT][G::KC], const uint8_t* kn,
                                          uint32_t (&pk)[G::KVC][QT][4], float (&m_run)[QT], float (&l_run)[QT],
                                          f32x4_t (&oacc)[G::DT][QT], float c2) {
  constexpr int C1 = (G::KC + 2) / 3, C2 = (2 * G::KC + 2) / 3;
  typename G::E::v8 kf[G::KC][G::MT];
#pragma unroll
  for (int c = 0; c < G::KC; ++c)
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
      kf[c][mt] = G::E::cast(*reinterpret_cast<const u32x4_t*>(kn + mt * 16 * G::KSTR + c * 64));
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int t = 0; t < QT; ++t) s_nxt[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mfmas = [&](int c0, int c1) __attribute__((always_inline)) {
#pragma unroll
    for (int c = c0; c < c1; ++c)
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int t = 0; t < QT; ++t)
          s_nxt[mt][t] = G::E::mfma(kf[c][mt], qf[t][c], s_nxt[mt][t]);
  };
  // phase 1: row max
  float mx[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    mx[t] = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[t] = fmaxf(mx[t], s_cur[mt][t][r]);
  }
  mfmas(0, C1);
  __builtin_amdgcn_sched_barrier(0);
  // phase 2: reductions across the row's four lanes, running max, rescale
  float m_neg[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float m_new = fmaxf(m_run[t], group_max(mx[t]) * c2);
    const bool moved = m_new > m_run[t] + kRescaleThreshold;
    const float alpha = moved ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;  // 0 when m_run = -inf
    m_run[t] = moved ? m_new : m_run[t];
    l_run[t] *= alpha;
#pragma unroll
    for (int i = 0; i < G::DT; ++i) oacc[i][t] *= alpha;
    m_neg[t] = (m_run[t] == -INFINITY) ? 0.f : -m_run[t];
  }
  mfmas(C1, C2);
  __builtin_amdgcn_sched_barrier(0);
  // phase 3: p = exp2(s c2 - m), row sums, P^T packed to bf16
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[mt][t][r], c2, m_neg[t]));
        s_cur[mt][t][r] = pv;
        lsum += pv;
      }
    l_run[t] += lsum;
#pragma unroll
    for (int kc = 0; kc < G::KVC; ++kc) {
      pk[kc][t][0] = G::E::pack(s_cur[2 * kc][t][0], s_cur[2 * kc][t][1]);
      pk[kc][t][1] = G::E::pack(s_cur[2 * kc][t][2], s_cur[2 * kc][t][3]);
      pk[kc][t][2] = G::E::pack(s_cur[2 * kc + 1][t][0], s_cur[2 * kc + 1][t][1]);
      pk[kc][t][3] = G::E::pack(s_cur[2 * kc + 1][t][2], s_cur[2 * kc + 1][t][3]);
    }
  }
  mfmas(C2, G::KC);
}

// Causal: keys a row block may attend, as planned on the host for the full
// key buffer -- up to the diagonal key of the block's last row, with the
// last query aligned to the last key (offset coff = Sk - Sq) -- clamped to
// [0, Sk].  Grids and split counts come from this bound; inside a block the
// range is narrowed to the valid keys (offset seqused_k - Sq).
__host__ __device__ __forceinline__ int causal_kmax(int rb, int rows, int Mp, int g, int coff, int Sk) {
  const int last_row = ((rb + 1) * rows < Mp ? (rb + 1) * rows : Mp) - 1;
  const int k = last_row / g + coff + 1;
  return k < 0 ? 0 : (k > Sk ? Sk : k);
}

// Causal grids: workgroup x takes row block nrb - 1 - x / zmax (heaviest
// first) and key range x % zmax of it (zmax = 1 without splitting).  Returns
// false for a key range past the block's last planned key: such a workgroup
// has no work, and the merge reads no partial from it.
template <bool SPLIT>
__device__ __forceinline__ bool causal_item(const FwdParams& p, int rows, int g, int& rb, int& z, int& kmax) {
  const int nrb = (p.Mp + rows - 1) / rows;
  const int x = blockIdx.x;
  const int q = SPLIT ? x / p.zmax : x;
  rb = nrb - 1 - q;
  z = SPLIT ? x - q * p.zmax : 0;
  kmax = causal_kmax(rb, rows, p.Mp, g, p.coff, p.Sk);
  return !SPLIT || z * p.kps < kmax;
}

// Element offset b*sb + r*ss + h*sh of a (batch, position, head) view.
// Indices and strides are non-negative and the host keeps the position and
// head strides below 2^31, so those two terms are 32x32-bit products; only
// the batch term takes a 64-bit stride.
__device__ __forceinline__ uint64_t view_off(int b, int r, int h, long long sb, long long ss, long long sh) {
  return (uint64_t)(uint32_t)b * (uint64_t)sb + (uint64_t)(uint32_t)r * (uint32_t)ss +
         (uint64_t)(uint32_t)h * (uint32_t)sh;
}

// Rows and keys of batch entry b.  Fixed shape: query positions 0..Sq-1
// and keys 0..n-1, n from seqused_k.  Packed variable-length batch: the
// b-th sequence, its offsets read on the device and clamped into the
// tensors (start in [0, total], end in [start, total], length at most the
// planned maximum), so any values stay in bounds.
struct Seq {
  int q0, sq;       // first query position, query count
  int k0, nk;       // first key position, attended key count
  long long lse0;   // lse index of (head 0, query 0); heads are p.lse_hs apart
};

__device__ __forceinline__ Seq seq_of(const FwdParams& p, int b) {
  Seq r;
  r.q0 = 0;
  r.sq = p.Sq;
  r.k0 = 0;
  r.nk = p.Sk;
  // The fixed-shape path falls straight through: a taken branch this early
  // costs an instruction-cache miss before the first tile copy is issued.
  if (__builtin_expect(p.cu_q != nullptr, 0)) {
    int a = min(max(p.cu_q[b], 0), p.total_q), e = min(max(p.cu_q[b + 1], a), p.total_q);
    r.q0 = a;
    r.sq = min(e - a, p.Sq);
    a = min(max(p.cu_k[b], 0), p.total_k);
    e = min(max(p.cu_k[b + 1], a), p.total_k);
    r.k0 = a;
    r.nk = min(e - a, p.Sk);
  } else if (p.seqused != nullptr) {
    r.nk = min(max(p.seqused[b], 0), p.Sk);
  }
  // uniform per workgroup: keeps buffer resources and loop bounds scalar
  r.q0 = __builtin_amdgcn_readfirstlane(r.q0);
  r.sq = __builtin_amdgcn_readfirstlane(r.sq);
  r.k0 = __builtin_amdgcn_readfirstlane(r.k0);
  r.nk = __builtin_amdgcn_readfirstlane(r.nk);
  r.lse0 = (long long)b * p.lse_bs + r.q0;  // one of the two terms is zero
  return r;
}

struct RowBlock {
  int rb;      // row block index
  int z;       // key chunk (split) index
  int kbeg, kend;
};

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
    blk.kend = min(min(blk.kend, nvalid), (min((rb + 1) * G::ROWS_WG, Mp) - 1) / g + (nvalid - sq.sq) + 1);
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
  const int s_lo = min(rw0, Mp - 1) / g + doff;
  const int s_hi = (min(rw0 + 16 * QT, Mp) - 1) / g + doff;

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
    const int s = ok ? r / g : 0;
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
      const int s = r / g, hh = r - s * g;
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
template <int D, int QT, int KW, int BN, bool CAUSAL, bool SPLIT, int DTY, int OUTF>
__global__ void __launch_bounds__(KW * 64, 1)
fwd_ks_kernel(const FwdParams p) {
  using G = Geo<D, QT, 1, BN, DTY>;  // per-wave geometry: one wave issues its own tile copies
  constexpr int ROWS = 16 * QT;
  pin_params(p);
  static_assert(!G::TRASH, "per-wave tiles must be whole 64-slot windows");
  // LDS: KW per-wave K/V buffers, then the workgroup's Q tile (rows at the K
  // stride, read like K fragments); after the main loop the same memory is
  // the merge area.
  constexpr int Q_INSTR = round_up(ROWS * (G::KSTR / 16), 64) / 64;  // 1 KiB copies of the Q tile
  constexpr int Q_OFF = KW * G::STAGE_B;
  constexpr int OSTR = D * 4 + 16;                       // merge area: bytes per O row (padded)
  constexpr int MERGE_B = KW * ROWS * OSTR + KW * ROWS * 8;
  constexpr int TILE_B = Q_OFF + Q_INSTR * 1024;
  constexpr int LDS_B = TILE_B > MERGE_B ? TILE_B : MERGE_B;
  static_assert(LDS_B <= 160 * 1024, "LDS of one workgroup");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level addresses stay scalar
  const int col = lane & 15, grp = lane >> 4;
  const int bh = blockIdx.y;
  const int b = udiv(bh, p.Hkv, p.hkv_m), hk = bh - b * p.Hkv;
  const int g = p.g;

  const Seq sq = seq_of(p, b);
  const int nvalid = sq.nk;
  const int Mp = sq.sq * g;  // packed rows of this batch entry (the grid covers the planned maximum)

  RowBlock blk;
  if constexpr (CAUSAL) {
    int rb, item, kmax;
    if (!causal_item<SPLIT>(p, ROWS, g, rb, item, kmax)) return;
    blk.rb = rb;
    blk.z = item;
    blk.kbeg = SPLIT ? item * p.kps : 0;
    blk.kend = SPLIT ? min(blk.kbeg + p.kps, kmax) : kmax;
    // the valid keys, up to the diagonal of the block's last row
    blk.kend = min(min(blk.kend, nvalid), (min((rb + 1) * ROWS, Mp) - 1) / g + (nvalid - sq.sq) + 1);
  } else {
    blk.rb = blockIdx.x;
    blk.z = SPLIT ? blockIdx.z : 0;
    blk.kbeg = SPLIT ? blk.z * p.kps : 0;
    blk.kend = SPLIT ? min(blk.kbeg + p.kps, nvalid) : nvalid;
  }
  const int row0 = blk.rb * ROWS;
  if (row0 >= Mp) return;  // past a shorter sequence of a packed batch: nothing to do
  const int kbeg = blk.kbeg, kend = blk.kend;
  const int doff = CAUSAL ? nvalid - sq.sq : 0;  // causal: diagonal key offset (last query <-> last valid key)
  const int s_lo = min(row0, Mp - 1) / g + doff;

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
  uint8_t* kbuf = smem + wave * G::STAGE_B;
  uint8_t* vbuf = kbuf + G::K_B;
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

  // Q tile: packed rows row0 .. row0+ROWS-1, copied once per workgroup
  // (wave w issues copies w, w+KW, ...) into LDS at the K row stride.  The
  // buffer starts at the block's first position; rows past Mp and the row
  // padding read as zeros.
  {
    const int s_first = row0 / g;
    const int s_last = (min(row0 + ROWS, Mp) - 1) / g;
    const uint32_t qrow_b = (uint32_t)(p.q_ss * 2), qhead_b = (uint32_t)(p.q_sh * 2);
    const u32x4_t rq = make_rsrc(p.q + view_off(b, sq.q0 + s_first, hk * g, p.q_sb, p.q_ss, p.q_sh),
                                 (uint32_t)(s_last - s_first) * qrow_b + (uint32_t)(g - 1) * qhead_b + D * 2);
    const uint32_t lds_q = (uint32_t)(uintptr_t)(lds_void_t*)(smem + Q_OFF);
    for (int j = wave; j < Q_INSTR; j += KW) {
      const int P = j * 64 + lane;
      const int row = P / (G::KSTR / 16), ch = P - row * (G::KSTR / 16);
      const int r = row0 + row;
      uint32_t off = kOutOfRange;
      if (row < ROWS && ch < G::CPR && r < Mp) {
        const int sq = r / g;
        off = (uint32_t)(sq - s_first) * qrow_b + (uint32_t)(r - sq * g) * qhead_b + (uint32_t)(ch * 16);
      }
      copy16_to_lds(rq, off, __builtin_amdgcn_readfirstlane(lds_q + j * 1024));
    }
  }
  // First K and V tiles after Q: waiting for all but the V copies then means
  // Q and K have landed, and the first QK^T overlaps the V copies.
  if (nown > 0) {
    issue_k(kbeg + wave * BN);
    issue_v(kbeg + wave * BN);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(G::LPT_V));
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
    srow[t] = r < Mp ? r / g + doff : -1;  // causal: the row's diagonal key
#pragma unroll
    for (int c = 0; c < G::KC; ++c) {
      qf[t][c] = G::E::cast(*reinterpret_cast<const u32x4_t*>(smem + Q_OFF + (16 * t + col) * G::KSTR + c * 64 + grp * 16));
    }
  }

  uint32_t k_lane, v_lane;
  lane_bases<G>(lane, k_lane, v_lane);
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
  float l_tot[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) l_tot[t] = group_sum(l_run[t]);
  __syncthreads();  // every wave is done with its tiles: the LDS becomes the merge area
  float* mls = reinterpret_cast<float*>(smem + KW * ROWS * OSTR);  // [row][wave] (m, l)
  {
    uint8_t* ob = smem + wave * ROWS * OSTR;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int rl = 16 * t + col;
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        if (d < D) *reinterpret_cast<f32x4_t*>(ob + rl * OSTR + d * 4) = oacc[dt][t];
      }
      if (grp == 0) *reinterpret_cast<u32x2_t*>(mls + 2 * (rl * KW + wave)) =
          u32x2_t{__float_as_uint(m_run[t]), __float_as_uint(l_tot[t])};
    }
  }
  __syncthreads();
  constexpr int TPR = KW * 64 / ROWS;  // threads per row
  static_assert(TPR * ROWS == KW * 64, "whole rows per workgroup pass");
  const int rl = tid / TPR, c0 = tid - rl * TPR;
  const int r = row0 + rl;
  if (r < Mp) {
    float mw[KW], fw[KW];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      mw[w] = mls[2 * (rl * KW + w)];
      fw[w] = mls[2 * (rl * KW + w) + 1];  // l of wave w
      if (fw[w] > 0.f) M = fmaxf(M, mw[w]);
    }
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
    const int s = r / g, hh = r - s * g;
#pragma unroll
    for (int j = 0; j < (G::CPR + TPR - 1) / TPR; ++j) {
      const int ch = c0 + TPR * j;
      if (ch < G::CPR) {
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const uint8_t* src = smem + (w * ROWS + rl) * OSTR + ch * 32;
          a0 += fw[w] * *reinterpret_cast<const f32x4_t*>(src);
          a1 += fw[w] * *reinterpret_cast<const f32x4_t*>(src + 16);
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
    nz = (causal_kmax(rb, ROWS_WG, p.Mp, g, p.coff, p.Sk) + p.kps - 1) / p.kps;
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
  const int s = r / g, hh = r - s * g;
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

template <int D, int QT, int KW, int BN, bool CAUSAL, bool SPLIT, int DTY, int OUTF = kOutElem>
static hipError_t launch_ks_variant(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  constexpr int ROWS = 16 * QT;
  const int nrb = (p.Mp + ROWS - 1) / ROWS;
  dim3 grid;
  if (CAUSAL) {
    grid = dim3((unsigned)(nrb * (SPLIT ? std::max(p.zmax, 1) : 1)), p.B * p.Hkv, 1);
  } else {
    grid = dim3(nrb, p.B * p.Hkv, SPLIT ? plan.nsplit : 1);
  }
  hipLaunchKernelGGL((fwd_ks_kernel<D, QT, KW, BN, CAUSAL, SPLIT, DTY, OUTF>), grid, dim3(KW * 64), 0, stream, p);
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
// same rows), keys per tile.  Every variant is built with and without causal
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

#define FA_KS_VARIANTS(X)  \
  X(kBf16, 64, 2, 4, 64)   \
  X(kBf16, 72, 2, 4, 64)   \
  X(kBf16, 256, 2, 4, 32)  \
  X(kBf16, 256, 1, 4, 32)  \
  X(kBf16, 256, 2, 2, 32)  \
  X(kF16, 256, 2, 4, 32)   \
  X(kF16, 256, 1, 4, 32)

// (nw, kw) of a plan: kw == 1, waves on different rows; kw == nw, every wave
// on the same rows (key-split kernel); otherwise kw key groups of nw / kw
// waves each (row-split kernel).
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
  if (nst != 1) return false;
#define FA_KS_MATCH(t_, d_, q_, k_, b_) \
  if (dtype == t_ && D == d_ && qt == q_ && kw == k_ && bn == b_) return true;
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
                               l.nst == 1));
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
  return plan.qt == 1 ? launch_ks_variant<256, 1, 4, 32, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream)
                      : launch_ks_variant<256, 2, 4, 32, CAUSAL, SPLIT, kBf16, kOutNvfp4>(p, plan, stream);
}

hipError_t launch_fwd(const FwdParams& p, const LaunchPlan& plan, hipStream_t stream) {
  if (plan.outf == kOutNvfp4) {
    if (!nvfp4_variant_exists(plan)) return hipErrorInvalidValue;
    if (plan.causal)
      return plan.split ? launch_nvfp4<true, true>(p, plan, stream) : launch_nvfp4<true, false>(p, plan, stream);
    return plan.split ? launch_nvfp4<false, true>(p, plan, stream) : launch_nvfp4<false, false>(p, plan, stream);
  }
  if (plan.kw > 1 && plan.kw == plan.nw) {
#define FA_KS_DISPATCH(t_, d_, q_, k_, b_)                                                          \
  if (plan.dtype == t_ && plan.D == d_ && plan.qt == q_ && plan.kw == k_ && plan.bn == b_) {         \
    if (plan.causal)                                                                                \
      return plan.split ? launch_ks_variant<d_, q_, k_, b_, true, true, t_>(p, plan, stream)        \
                        : launch_ks_variant<d_, q_, k_, b_, true, false, t_>(p, plan, stream);      \
    return plan.split ? launch_ks_variant<d_, q_, k_, b_, false, true, t_>(p, plan, stream)         \
                      : launch_ks_variant<d_, q_, k_, b_, false, false, t_>(p, plan, stream);       \
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
