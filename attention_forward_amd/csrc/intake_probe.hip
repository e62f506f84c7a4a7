// Intake ceiling of one compute unit on gfx950: how many bytes per clock a
// compute unit takes in from L2 when every compute unit streams at once.
//
// This bounds the K/V streaming of the attention kernels: a workgroup that
// owns a block of query rows must bring every K and V byte of its key range
// into its compute unit, through the same path this probe measures (buffer
// loads that write LDS directly, and, for comparison, coalesced loads into
// registers).  Each workgroup streams the same 1 MiB source (resident in L2
// after the first pass) PASSES times, four waves each keeping 15 KiB of
// copies in flight, and records its elapsed shader clocks.  Prints one JSON
// line: bytes per clock per compute unit (median over the compute units) and
// the shader clock seen while streaming.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

#define PROBE_CHECK(x)                                                                 \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "intake_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                         \
    }                                                                                  \
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

constexpr int kWaves = 4;
constexpr int kSlots = 16;  // 1 KiB LDS slots per wave

// MODE 0: buffer loads into LDS; MODE 1: coalesced 16-byte loads into registers.
template <int MODE>
__global__ void __launch_bounds__(kWaves * 64) stream(const uint8_t* src, uint32_t bytes, int passes,
                                                      unsigned long long* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves * kSlots * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunks = (int)(bytes / 1024);
  const unsigned long long t0 = __builtin_readcyclecounter();
  u32x4_t acc = {0u, 0u, 0u, 0u};
  if (MODE == 0) {
    const u32x4_t rs = make_rsrc(src, bytes);
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)ring + wave * kSlots * 1024;
    int n = 0;
    for (int p = 0; p < passes; ++p)
      for (int c = wave; c < chunks; c += kWaves) {
        copy16_to_lds(rs, (uint32_t)c * 1024 + lane * 16, base + (n % kSlots) * 1024);
        ++n;
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (15 << 8));  // vmcnt(15): 15 KiB in flight per wave
      }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  } else {
    for (int p = 0; p < passes; ++p)
      for (int c0 = wave; c0 < chunks; c0 += 8 * kWaves) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = min(c0 + u * kWaves, chunks - 1);
          v[u] = *reinterpret_cast<const u32x4_t*>(src + (size_t)c * 1024 + lane * 16);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
      }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_readcyclecounter();
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
  if (acc[0] == 0x12345678u) sink[0] = acc[1];  // keeps the register loads
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  PROBE_CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const uint32_t bytes = 1u << 20;
  const int passes = 16;
  uint8_t* src = nullptr;
  unsigned long long* cyc = nullptr;
  uint32_t* sink = nullptr;
  PROBE_CHECK(hipMalloc(&src, bytes));
  PROBE_CHECK(hipMemset(src, 1, bytes));
  PROBE_CHECK(hipMalloc(&cyc, sizeof(unsigned long long) * cus));
  PROBE_CHECK(hipMalloc(&sink, 16));
  hipEvent_t e0, e1;
  PROBE_CHECK(hipEventCreate(&e0));
  PROBE_CHECK(hipEventCreate(&e1));
  std::vector<unsigned long long> h(cus);
  double rate[2], mhz[2];
  for (int mode = 0; mode < 2; ++mode) {
    for (int rep = 0; rep < 2; ++rep) {  // the first run warms L2 and the clocks
      PROBE_CHECK(hipEventRecord(e0));
      if (mode == 0)
        hipLaunchKernelGGL(stream<0>, dim3(cus), dim3(kWaves * 64), 0, 0, src, bytes, passes, cyc, sink);
      else
        hipLaunchKernelGGL(stream<1>, dim3(cus), dim3(kWaves * 64), 0, 0, src, bytes, passes, cyc, sink);
      PROBE_CHECK(hipGetLastError());
      PROBE_CHECK(hipEventRecord(e1));
      PROBE_CHECK(hipEventSynchronize(e1));
    }
    float ms = 0.f;
    PROBE_CHECK(hipEventElapsedTime(&ms, e0, e1));
    PROBE_CHECK(hipMemcpy(h.data(), cyc, sizeof(unsigned long long) * cus, hipMemcpyDeviceToHost));
    std::sort(h.begin(), h.end());
    const double med = (double)h[cus / 2];
    rate[mode] = (double)bytes * passes / med;
    mhz[mode] = (double)h[cus - 1] / (ms * 1e3);  // slowest compute unit's clocks over the event time
  }
  printf("{\"compute_units\": %d, \"lds_stream_bytes_per_clk_per_cu\": %.2f, \"vgpr_load_bytes_per_clk_per_cu\": %.2f, "
         "\"shader_mhz_lds\": %.0f, \"shader_mhz_vgpr\": %.0f}\n",
         cus, rate[0], rate[1], mhz[0], mhz[1]);
  return 0;
}
