// Device-side modular arithmetic and the ChaCha block for gfx950.
//
// Residues are canonical uint32 values below a prime r < 2^31 (the 32-bit RNS
// chain of the Perseus runtime, its opening paragraph on the 32-bit FIDESlib
// port). Three reductions are used, chosen from measured gfx950 instruction
// rates (32-bit multiplies issue at close to the full VALU rate):
//   * Shoup multiplication by a constant w with companion floor(w 2^32 / r):
//     mul_hi, mul_lo, mad_u64_u32, add, min -- five instructions;
//   * Montgomery reduction (REDC) of a 64-bit sum x < r 2^32, giving
//     x 2^-32 mod r; two products of residues may be summed before one REDC;
//   * add/sub with one unsigned-min correction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pc {

__device__ __forceinline__ uint32_t add_mod(uint32_t a, uint32_t b, uint32_t r) {
  const uint32_t s = a + b;  // < 2r < 2^32
  return min(s, s - r);
}

__device__ __forceinline__ uint32_t sub_mod(uint32_t a, uint32_t b, uint32_t r) {
  const uint32_t d = a - b;  // wraps when a < b; d + r is then the answer
  return min(d, d + r);
}

// Reduce x in [0, 2r) to [0, r).
__device__ __forceinline__ uint32_t reduce_2r(uint32_t x, uint32_t r) { return min(x, x - r); }

// x * w mod r for any 32-bit x, w < r, wp = floor(w 2^32 / r). Result canonical.
__device__ __forceinline__ uint32_t mul_shoup(uint32_t x, uint32_t w, uint32_t wp, uint32_t r) {
  const uint32_t qh = __umulhi(x, wp);
  const uint32_t t = x * w - qh * r;  // in [0, 2r)
  return min(t, t - r);
}

// Montgomery reduction: x < r 2^32  ->  x 2^-32 mod r, canonical.
// rinv_neg = -r^-1 mod 2^32.
__device__ __forceinline__ uint32_t redc(uint64_t x, uint32_t r, uint32_t rinv_neg) {
  const uint32_t m = (uint32_t)x * rinv_neg;
  const uint64_t s = x + (uint64_t)m * r;  // x + m r < 2 r 2^32 < 2^64, divisible by 2^32
  const uint32_t t = (uint32_t)(s >> 32);  // < 2r
  return min(t, t - r);
}

__device__ __forceinline__ uint64_t mul_wide(uint32_t a, uint32_t b) { return (uint64_t)a * b; }

// acc = a b (first) and acc += a b (mac): one 32 x 32 + 64 -> 64 multiply-add
// each, written as the instruction itself so that the compiler cannot widen
// the operands to 64 bits ahead of a loop (a register pair per kept operand).
// The carry-out goes to a scratch scalar pair; the caller keeps acc + a b below
// 2^64.
__device__ __forceinline__ uint64_t mul_wide_op(uint32_t a, uint32_t b) {
  uint64_t acc, cc;
  asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(acc), "=s"(cc) : "v"(a), "v"(b));
  return acc;
}
__device__ __forceinline__ void mac_wide_op(uint64_t& acc, uint32_t a, uint32_t b) {
  uint64_t cc;
  asm("v_mad_u64_u32 %0, %1, %2, %3, %0" : "+v"(acc), "=s"(cc) : "v"(a), "v"(b));
}

// base[idx] addressed through a 32-bit byte offset (idx < 2^30): the compiler
// can then use a uniform 64-bit base plus a 32-bit per-lane offset instead of
// a full 64-bit address per lane.
template <class T>
__device__ __forceinline__ T& at32(T* base, uint32_t idx) {
  using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
  return *reinterpret_cast<T*>(reinterpret_cast<B*>(base) + (idx << 2));
}

// Streaming access for a word that this kernel touches once and no kernel
// reads again soon (the accumulators that an earlier launch wrote, the final
// output): the non-temporal hint keeps it from evicting reused lines.
__device__ __forceinline__ uint32_t load_stream(const uint32_t* base, uint32_t idx) {
  return __builtin_nontemporal_load(&at32(base, idx));
}
__device__ __forceinline__ void store_stream(uint32_t* base, uint32_t idx, uint32_t v) {
  __builtin_nontemporal_store(v, &at32(base, idx));
}

// x w 2^-32 mod r for any 32-bit x and w < r, canonical: with w a twiddle in
// Montgomery form (w0 2^32 mod r) this is x w0 mod r.
__device__ __forceinline__ uint32_t mul_mont(uint32_t x, uint32_t w, uint32_t r, uint32_t rinv_neg) {
  return redc(mul_wide(x, w), r, rinv_neg);
}

__device__ __forceinline__ uint32_t bitrev(uint32_t x, int bits) {
  return bits ? (__builtin_bitreverse32(x) >> (32 - bits)) : 0u;
}

// ---------------------------------------------------------------------------
// ChaCha block (Bernstein's ChaCha; state layout of RFC 8439): constants,
// 8 key words, block counter in word 12, nonce in words 13..15. ROUNDS is the
// number of rounds (12 for the key expander; 20 only to compare with ChaCha20).
// ---------------------------------------------------------------------------

struct ChaChaKey {
  uint32_t k[8];
};

__device__ __forceinline__ uint32_t rotl32(uint32_t x, int n) { return __builtin_rotateleft32(x, n); }

#define PC_QR(a, b, c, d)      \
  a += b;                      \
  d = rotl32(d ^ a, 16);       \
  c += d;                      \
  b = rotl32(b ^ c, 12);       \
  a += b;                      \
  d = rotl32(d ^ a, 8);        \
  c += d;                      \
  b = rotl32(b ^ c, 7);

template <int ROUNDS>
__device__ __forceinline__ void chacha_block(const ChaChaKey& key, uint32_t counter, uint32_t n0, uint32_t n1,
                                             uint32_t n2, uint32_t out[16]) {
  const uint32_t c0 = 0x61707865u, c1 = 0x3320646eu, c2 = 0x79622d32u, c3 = 0x6b206574u;
  uint32_t x0 = c0, x1 = c1, x2 = c2, x3 = c3;
  uint32_t x4 = key.k[0], x5 = key.k[1], x6 = key.k[2], x7 = key.k[3];
  uint32_t x8 = key.k[4], x9 = key.k[5], x10 = key.k[6], x11 = key.k[7];
  uint32_t x12 = counter, x13 = n0, x14 = n1, x15 = n2;
#pragma unroll
  for (int i = 0; i < ROUNDS / 2; ++i) {
    PC_QR(x0, x4, x8, x12)
    PC_QR(x1, x5, x9, x13)
    PC_QR(x2, x6, x10, x14)
    PC_QR(x3, x7, x11, x15)
    PC_QR(x0, x5, x10, x15)
    PC_QR(x1, x6, x11, x12)
    PC_QR(x2, x7, x8, x13)
    PC_QR(x3, x4, x9, x14)
  }
  out[0] = x0 + c0;
  out[1] = x1 + c1;
  out[2] = x2 + c2;
  out[3] = x3 + c3;
  out[4] = x4 + key.k[0];
  out[5] = x5 + key.k[1];
  out[6] = x6 + key.k[2];
  out[7] = x7 + key.k[3];
  out[8] = x8 + key.k[4];
  out[9] = x9 + key.k[5];
  out[10] = x10 + key.k[6];
  out[11] = x11 + key.k[7];
  out[12] = x12 + counter;
  out[13] = x13 + n0;
  out[14] = x14 + n1;
  out[15] = x15 + n2;
}

#undef PC_QR

// (lo + 2^32 hi) mod r, returned in Montgomery form (times 2^-32). hi is first
// reduced below r (r > 2^30, so hi < 4r needs at most three corrections); then
// x = 2^32 h + lo <= r 2^32 - 1 is a valid REDC input.
__device__ __forceinline__ uint32_t word_pair_to_mont(uint32_t lo, uint32_t hi, uint32_t r, uint32_t rinv_neg) {
  uint32_t h = min(hi, hi - r);
  h = min(h, h - r);
  h = min(h, h - r);
  return redc(((uint64_t)h << 32) | lo, r, rinv_neg);
}

}  // namespace pc
