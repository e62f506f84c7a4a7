// Intake ceiling of one compute unit on gfx950: how many bytes per clock a
// compute unit takes in from L2 when every compute unit streams at once.
//
// This bounds the K/V streaming of the attention kernels: a workgroup that
// owns a block of query rows must bring every K and V byte of its key range
// into its compute unit, through the path this probe measures (buffer loads
// that write LDS directly, and, for comparison, coalesced loads into
// registers).  One workgroup per compute unit streams an L2-resident 1 MiB
// source, each active wave keeping 15 KiB of copies in flight, and records
// its elapsed shader clocks.  Every compute unit walks the source in the
// same order, the waves of one compute unit on neighbouring 1 KiB chunks, so
// the requests of any moment fall on one 4 KiB block: the worst case for
// the spread over L2 channels (waves on blocks of their own do better).
// Cases:
//   lds_1k:     each copy reads 1 KiB contiguous, four waves;
//   lds_rows:   each copy reads 64 bytes of each of 16 rows 512 bytes apart
//               (the attention kernels' K/V piece copies), four waves;
//   lds_rows_1w: the same with one wave per compute unit;
//   lds_lines:  each copy reads 128 bytes of each of 8 rows 512 bytes apart
//               (whole cache lines), four waves;
//   lds_lines_1w: the same with one wave per compute unit;
//   vgpr_1k:    coalesced 16-byte register loads, 1 KiB per instruction.
// Prints one JSON line: bytes per clock per compute unit (median over the
// compute units) per case, and the shader clock seen while streaming.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

#define PROBE_CHECK(x)                                                                   \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      fprintf(stderr, "intake_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                           \
    }                                                                                    \
  } while (0)

__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(u32x4_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int kSlots = 16;  // 1 KiB LDS slots per wave
constexpr uint32_t kBytes = 1u << 20;

// MODE 0: 1 KiB contiguous copies into LDS; MODE 1: 16 rows x 64 bytes per
// copy into LDS; MODE 2: coalesced 16-byte loads into registers; MODE 3: 8
// rows x 128 bytes per copy into LDS.  NW waves
// of the workgroup stream (the others return at once).
template <int MODE, int NW>
__global__ void __launch_bounds__(256) stream(const uint8_t* src, int passes, unsigned long long* cycles,
                                              uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4 * kSlots * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= NW) return;
  // chunk c of the source: MODE 0 / 2 bytes [1024c, 1024c + 1024); MODE 1
  // 64-byte column (c % 8) of rows 16(c / 8) .. +15 of 512-byte rows; MODE 3
  // 128-byte column (c % 4) of rows 8(c / 4) .. +7
  const int chunks = (int)(kBytes / 1024);
  const uint32_t lane_off = MODE == 1   ? (uint32_t)(lane >> 2) * 512 + (uint32_t)(lane & 3) * 16
                            : MODE == 3 ? (uint32_t)(lane >> 3) * 512 + (uint32_t)(lane & 7) * 16
                                        : (uint32_t)lane * 16;
  auto chunk_off = [](int c) -> uint32_t {
    return MODE == 1   ? (uint32_t)(c >> 3) * 8192 + (uint32_t)(c & 7) * 64
           : MODE == 3 ? (uint32_t)(c >> 2) * 4096 + (uint32_t)(c & 3) * 128
                       : (uint32_t)c * 1024;
  };
  const unsigned long long t0 = __builtin_readcyclecounter();
  u32x4_t acc = {0u, 0u, 0u, 0u};
  if (MODE != 2) {
    const u32x4_t rs = make_rsrc(src, kBytes);
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)ring + wave * kSlots * 1024;
    int n = 0;
    for (int p = 0; p < passes; ++p)
      for (int c = wave; c < chunks; c += NW) {
        copy16_to_lds(rs, lane_off + chunk_off(c), base + (n % kSlots) * 1024);
        ++n;
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (15 << 8));  // vmcnt(15): 15 KiB in flight per wave
      }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  } else {
    for (int p = 0; p < passes; ++p)
      for (int c0 = wave; c0 < chunks; c0 += 8 * NW) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = min(c0 + u * NW, chunks - 1);
          v[u] = *reinterpret_cast<const u32x4_t*>(src + (size_t)c * 1024 + lane * 16);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
      }
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
  if (acc[0] == 0x12345678u) sink[0] = acc[1];  // keeps the register loads
}

struct Result {
  double bytes_per_clk, mhz;
};

template <int MODE, int NW>
Result run(const uint8_t* src, unsigned long long* cyc, uint32_t* sink, int cus, hipEvent_t e0, hipEvent_t e1) {
  const int passes = 16;
  std::vector<unsigned long long> h(cus);
  for (int rep = 0; rep < 2; ++rep) {  // the first run warms L2 and the clocks
    PROBE_CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL((stream<MODE, NW>), dim3(cus), dim3(256), 0, 0, src, passes, cyc, sink);
    PROBE_CHECK(hipGetLastError());
    PROBE_CHECK(hipEventRecord(e1));
    PROBE_CHECK(hipEventSynchronize(e1));
  }
  float ms = 0.f;
  PROBE_CHECK(hipEventElapsedTime(&ms, e0, e1));
  PROBE_CHECK(hipMemcpy(h.data(), cyc, sizeof(unsigned long long) * cus, hipMemcpyDeviceToHost));
  std::sort(h.begin(), h.end());
  return Result{(double)kBytes * passes / (double)h[cus / 2], (double)h[cus - 1] / (ms * 1e3)};
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  PROBE_CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  uint8_t* src = nullptr;
  unsigned long long* cyc = nullptr;
  uint32_t* sink = nullptr;
  PROBE_CHECK(hipMalloc(&src, kBytes));
  PROBE_CHECK(hipMemset(src, 1, kBytes));
  PROBE_CHECK(hipMalloc(&cyc, sizeof(unsigned long long) * cus));
  PROBE_CHECK(hipMalloc(&sink, 16));
  hipEvent_t e0, e1;
  PROBE_CHECK(hipEventCreate(&e0));
  PROBE_CHECK(hipEventCreate(&e1));
  const Result a = run<0, 4>(src, cyc, sink, cus, e0, e1);
  const Result b = run<1, 4>(src, cyc, sink, cus, e0, e1);
  const Result c = run<1, 1>(src, cyc, sink, cus, e0, e1);
  const Result d = run<2, 4>(src, cyc, sink, cus, e0, e1);
  const Result e = run<3, 4>(src, cyc, sink, cus, e0, e1);
  const Result f = run<3, 1>(src, cyc, sink, cus, e0, e1);
  printf("{\"compute_units\": %d, \"bytes_per_clk_per_cu\": {\"lds_1k\": %.2f, \"lds_rows\": %.2f, \"lds_rows_1w\": %.2f, "
         "\"lds_lines\": %.2f, \"lds_lines_1w\": %.2f, \"vgpr_1k\": %.2f}, \"shader_mhz\": %.0f}\n",
         cus, a.bytes_per_clk, b.bytes_per_clk, c.bytes_per_clk, e.bytes_per_clk, f.bytes_per_clk, d.bytes_per_clk, b.mhz);
  return 0;
}
