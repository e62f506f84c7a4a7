// Device-side building blocks of the kernels in fa_kernels.hip: element
// types, NVFP4 coding, tile copies, the tile geometry, the S^T / softmax /
// O^T phases of one tile, and the mapping of workgroups to rows and keys.
// Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// s_waitcnt with lgkmcnt = n (0..15; larger waits for none) and vmcnt /
// expcnt at their maxima.  The immediate must be a constant: in an unrolled
// loop n is one, and the switch folds to a single instruction.
constexpr int waitcnt_lgkm(int n) { return 15 | (3 << 14) | (7 << 4) | (n << 8); }
__device__ __forceinline__ void wait_lgkm(int n) {
  switch (n) {
#define FA_WAIT_LGKM(n_)                                   \
  case n_:                                                 \
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(n_));          \
    break;
    FA_WAIT_LGKM(0) FA_WAIT_LGKM(1) FA_WAIT_LGKM(2) FA_WAIT_LGKM(3) FA_WAIT_LGKM(4) FA_WAIT_LGKM(5)
    FA_WAIT_LGKM(6) FA_WAIT_LGKM(7) FA_WAIT_LGKM(8) FA_WAIT_LGKM(9) FA_WAIT_LGKM(10) FA_WAIT_LGKM(11)
    FA_WAIT_LGKM(12) FA_WAIT_LGKM(13) FA_WAIT_LGKM(14)
#undef FA_WAIT_LGKM
    default:
      break;
  }
}

// s_waitcnt with vmcnt = n (0..63), for counts that are constants only after
// unrolling (the switch then folds to one instruction).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define FA_WAIT_VM(n_)                                \
  case n_:                                            \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(n_));       \
    break;
#define FA_WAIT_VM8(b_) FA_WAIT_VM(b_) FA_WAIT_VM(b_ + 1) FA_WAIT_VM(b_ + 2) FA_WAIT_VM(b_ + 3) \
  FA_WAIT_VM(b_ + 4) FA_WAIT_VM(b_ + 5) FA_WAIT_VM(b_ + 6) FA_WAIT_VM(b_ + 7)
    FA_WAIT_VM8(0) FA_WAIT_VM8(8) FA_WAIT_VM8(16) FA_WAIT_VM8(24)
    FA_WAIT_VM8(32) FA_WAIT_VM8(40) FA_WAIT_VM8(48) FA_WAIT_VM8(56)
#undef FA_WAIT_VM8
#undef FA_WAIT_VM
    default:
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      break;
  }
}

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
// head) lands on the same XCD and its K/V is fetched into one L2 only, and
// each XCD takes a contiguous run of (batch, kv head) pairs: neighbouring
// heads share cache lines when a head row is not a multiple of 128 bytes
// (144 bytes at D72), so a line is then fetched by one XCD, not two.
// The grid sizes come from the launch parameters (nrb row blocks by B*Hkv),
// not from the dispatch packet, which would take two more dependent scalar
// loads before the first tile copy.
// n / d for 0 <= n < 2^31 and d >= 1, given m = floor((2^32 - 1) / d): the
// high half of n*m is the quotient or one less (m > (2^32 - 1) / d - 1 and
// n < 2^31 keep the error of n*m / 2^32 below one), so one correction step
// makes it exact.  A multiply and a correction (scalar for uniform
// operands, vector otherwise), where the compiler's division by a runtime
// value takes a float reciprocal and about 30 more instructions.
__device__ __forceinline__ int udiv(int n, int d, uint32_t m) {
  const uint32_t q = __umulhi((uint32_t)n, m);
  return (int)(q + ((uint32_t)n - q * (uint32_t)d >= (uint32_t)d ? 1u : 0u));
}

// Item of workgroup n in a grid of N: the dispatcher deals workgroups to
// the 8 XCDs in turn (n goes to XCD n % 8), and this gives each XCD one
// contiguous run of item indices (the first N % 8 XCDs one item more), so
// neighbouring items share an L2.  A bijection of [0, N).
__device__ __forceinline__ int xcd_run(int n, int N) {
  const int q = N >> 3, r = N & 7, x = n & 7, j = n >> 3;
  return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

__device__ __forceinline__ void xcd_block(const FwdParams& p, int& bh, int& rb) {
  bh = blockIdx.y;
  rb = blockIdx.x;
  const int nbh = p.B * p.Hkv;
  if ((nbh & 7) == 0) {
    const int n = blockIdx.x + p.nrb * blockIdx.y;  // dispatch order: XCD n % 8
    const int slot = n >> 3, grp = udiv(slot, p.nrb, p.nrb_m);
    bh = (n & 7) * (nbh >> 3) + grp;  // XCD x: pairs x*nbh/8 .. (x+1)*nbh/8 - 1
    rb = slot - grp * p.nrb;
  }
}

// Loads the launch parameters the prologue needs at kernel entry, together:
// the compiler would otherwise fetch the strides only after the first
// branch, one more scalar-memory round trip before the first tile copy.
__device__ __forceinline__ void pin_params(const FwdParams& p) {
  asm volatile("" ::"s"(p.q_sb), "s"(p.q_ss), "s"(p.q_sh), "s"(p.k_sb), "s"(p.k_ss), "s"(p.k_sh), "s"(p.v_sb),
               "s"(p.v_ss), "s"(p.v_sh), "s"(p.o_ss), "s"(p.o_sh), "s"(p.o_sb));
  asm volatile("" ::"s"(p.nrb), "s"(p.nrb_m), "s"(p.hkv_m), "s"(p.kps), "s"(p.coff), "s"(p.zmax), "s"(p.zmax_m), "s"(p.Mp),
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

// causal_kmax on the device, for launch parameters p (p.Mp >= 1).
__device__ __forceinline__ int causal_kmax_dev(const FwdParams& p, int rb, int rows) {
  const int last_row = min((rb + 1) * rows, p.Mp) - 1;
  const int k = udiv(last_row, p.g, p.g_m) + p.coff + 1;
  return k < 0 ? 0 : (k > p.Sk ? p.Sk : k);
}

// Causal grids: workgroup x takes row block nrb - 1 - x / zmax (heaviest
// first) and key range x % zmax of it (zmax = 1 without splitting).  Returns
// false for a key range past the block's last planned key: such a workgroup
// has no work, and the merge reads no partial from it.
// PAIRED (unsplit grids of one (batch, kv head) whose workgroups are all
// resident at once, two per compute unit): the first half of the grid takes the heavy blocks from the
// heaviest down, the second half the light ones from the lightest up, so
// workgroups x and x + nrb/2, which the dispatcher places in the same order
// over the compute units, together attend about the same number of keys on
// every compute unit.
template <bool SPLIT, bool PAIRED = false>
__device__ __forceinline__ bool causal_item(const FwdParams& p, int rows, int g, int& rb, int& z, int& kmax) {
  const int nrb = (p.Mp + rows - 1) / rows;
  const int x = blockIdx.x;
  int q = SPLIT ? udiv(x, p.zmax, p.zmax_m) : x;
  if constexpr (PAIRED && !SPLIT) {
    // (one (batch, kv head) and at most two workgroups per compute unit)
    if (gridDim.y == 1 && nrb <= 2 * kComputeUnits) {
      const int half = (nrb + 1) >> 1;
      if (x >= half) q = nrb - 1 - (x - half);
    }
  }
  rb = nrb - 1 - q;
  z = SPLIT ? x - q * p.zmax : 0;
  kmax = causal_kmax_dev(p, rb, rows);
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

// With read_seqused false the fixed-shape path leaves nk at Sk and the
// caller reads seqused_k later (seqused_count), after issuing work that
// does not depend on it.
__device__ __forceinline__ Seq seq_of(const FwdParams& p, int b, bool read_seqused = true) {
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
  } else if (read_seqused && p.seqused != nullptr) {
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

// Attended key count of batch entry b for a Seq taken with read_seqused
// false: seqused_k[b] clamped to [0, Sk] for a fixed-shape call with a
// seqused_k array, else the count seq_of already holds.
__device__ __forceinline__ int seqused_count(const FwdParams& p, int b, const Seq& sq) {
  if (p.cu_q != nullptr || p.seqused == nullptr) return sq.nk;
  return __builtin_amdgcn_readfirstlane(min(max(p.seqused[b], 0), p.Sk));
}

struct RowBlock {
  int rb;      // row block index
  int z;       // key chunk (split) index
  int kbeg, kend;
};

}  // namespace fa
