// Issue-rate probe for the 32-bit integer VALU instructions the key-switching
// kernels are made of (gfx950). Each kernel runs eight independent chains of
// one operation per thread; an empty asm after every step keeps the compiler
// from folding the chain, so the loop body is the operation itself. Run it
// under `rocprofv3 --pmc SQ_INSTS_VALU`: the issued instructions divided by the
// dispatch's duration, the 256 compute units and the 2.4 GHz peak clock give
// the rate in wave-instructions per CU per clock (1.0 = four SIMD16s, each
// taking 4 clocks per wave64 instruction).
//
// Build: hipcc -O3 --offload-arch=gfx950 -o rate_probe rate_probe.hip
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

constexpr int kChains = 8;
constexpr int kThreads = 256;

__device__ __forceinline__ void opaque(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void opaque64(uint64_t& x) { asm volatile("" : "+v"(x)); }

// OP 0 v_add_u32, 1 v_mul_lo_u32, 2 v_mul_hi_u32, 3 v_mad_u64_u32, 4 v_add3_u32,
// 5 v_min_u32, 6 v_xor_b32, 7 v_alignbit_b32 (rotate),
// 8 a Montgomery butterfly (the NTT's: 5 + 3 + 3 instructions)
template <int OP>
__global__ void __launch_bounds__(kThreads) k_probe(uint32_t* out, uint32_t k1, uint32_t k2, uint32_t r,
                                                     uint32_t rinv, int iters) {
  uint32_t x[kChains];
  uint64_t a[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    x[c] = threadIdx.x * 2654435761u + c * k1;
    a[c] = x[c];
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (OP == 0) {
        x[c] = x[c] + k1;
      } else if constexpr (OP == 1) {
        x[c] = x[c] * k1;
      } else if constexpr (OP == 2) {
        x[c] = __umulhi(x[c], k1);
      } else if constexpr (OP == 3) {
        a[c] = (uint64_t)(uint32_t)a[c] * k1 + a[c];
      } else if constexpr (OP == 4) {
        x[c] = x[c] + x[c ^ 1] + k2;  // three variable operands: one v_add3_u32
      } else if constexpr (OP == 5) {
        x[c] = min(x[c], k1);
      } else if constexpr (OP == 6) {
        x[c] = x[c] ^ k1;
      } else if constexpr (OP == 7) {
        x[c] = __builtin_rotateleft32(x[c], 7);
      } else {
        // butterfly on the pair (x[c], x[c ^ 1]) with twiddle k1 in Montgomery form
        if (c & 1) continue;
        const uint64_t pr = (uint64_t)x[c + 1] * k1;
        const uint32_t m = (uint32_t)pr * rinv;
        const uint32_t t0 = (uint32_t)((pr + (uint64_t)m * r) >> 32);
        const uint32_t t = min(t0, t0 - r);
        const uint32_t u = x[c];
        const uint32_t s = u + t, d = u - t;
        x[c] = min(s, s - r);
        x[c + 1] = min(d, d + r);
        opaque(x[c + 1]);
      }
      if constexpr (OP == 3)
        opaque64(a[c]);
      else
        opaque(x[c]);
    }
  }
  uint32_t sum = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c) sum += x[c] + (uint32_t)a[c] + (uint32_t)(a[c] >> 32);
  out[blockIdx.x * kThreads + threadIdx.x] = sum;
}

const char* const kNames[] = {"v_add_u32",  "v_mul_lo_u32", "v_mul_hi_u32",   "v_mad_u64_u32", "v_add3_u32",
                              "v_min_u32",  "v_xor_b32",    "v_alignbit_b32", "butterfly"};

template <int OP>
int run(uint32_t* out, int blocks, int iters) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  // r = the first 31-bit NTT prime for N = 2^16, rinv = -r^-1 mod 2^32
  const uint32_t r = 2147352577u;
  uint32_t inv = 1;
  for (int i = 0; i < 5; ++i) inv *= 2u - r * inv;
  hipLaunchKernelGGL(k_probe<OP>, dim3(blocks), dim3(kThreads), 0, 0, out, 0x9e3779b9u, 12345u, r, 0u - inv,
                     iters);  // warm-up
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL(k_probe<OP>, dim3(blocks), dim3(kThreads), 0, 0, out, 0x9e3779b9u, 12345u, r, 0u - inv,
                     iters);
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  const double ops = (double)blocks * kThreads / 64.0 * iters * (OP == 8 ? kChains / 2 : kChains);
  printf("%-16s %8.3f ms  %.3f target wave-instructions per CU per clock at 2.4 GHz (event timing)\n", kNames[OP],
         ms, ops / (ms * 1e-3) / (256.0 * 2.4e9) * (OP == 8 ? 11.0 : 1.0));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

}  // namespace

int main() {
  const int blocks = 256 * 8, iters = 4096;
  uint32_t* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kThreads * 4) != hipSuccess) return 1;
  int rc = 0;
  rc |= run<0>(out, blocks, iters);
  rc |= run<1>(out, blocks, iters);
  rc |= run<2>(out, blocks, iters);
  rc |= run<3>(out, blocks, iters);
  rc |= run<4>(out, blocks, iters);
  rc |= run<5>(out, blocks, iters);
  rc |= run<6>(out, blocks, iters);
  rc |= run<7>(out, blocks, iters);
  rc |= run<8>(out, blocks, iters);
  (void)hipFree(out);
  return rc;
}
