// HIP kernels for CKKS hybrid key switching on gfx950 and their launchers.
//
// Steps (Perseus README, 'Layout': NTT and key-switching kernels; 'What's
// inside': the a half regenerated in-kernel from a ChaCha12 seed):
//   ModUp   : k_modup_inv_blk + k_modup_inv_col   iNTT of c1, scaled by N^-1 (Q_d/q_i)^-1
//             k_modup_bconv                       fast base conversion fused into NTT pass 1
//             k_modup_fwd_blk                     NTT pass 2 -> ext (evaluation form)
//   IP      : k_inner_product, k_ip_regen         automorphism gather, ChaCha12 a half, both sums
//   ModDown : k_md_inv_blk + k_md_inv_col         iNTT of the special limbs, scaled by N^-1 (P/p_t)^-1
//             k_md_bconv                          base conversion P -> q_i fused into NTT pass 1
//             k_md_fwd_blk                        NTT pass 2 fused with (acc - z) P^-1 (+ phi(c0))
//             k_seg_copy                          c0 into the segment layout (one ciphertext under
//                                                 rotation keys; see seg_src_index)
// The per-limb passes take one limb per grid row (blockIdx.y), blockIdx.x
// walking its column/block tiles; the conversions and the gathering kernels
// use 1-D grids placed by XCD (xcd_unit, limb_xcd_decode).
#include <algorithm>
#include <mutex>

#include "internal.h"
#include "ntt_pass.h"

// The launchers fall into five groups (NTT and ModUp, inner product, fused
// ModUp/inner product, ModDown, HMult/BSGS/keygen). Built with PC_PART = 1..5
// this file holds one group, so that the groups compile in parallel and link
// into one library; built without it, it holds all five.
#ifdef PC_PART
#define PC_IN_PART(n) (PC_PART == (n))
#else
#define PC_IN_PART(n) 1
#endif

namespace pc {

// ---------------------------------------------------------------------------
// pass shapes per ring size: column pass 2^LRC points (E = 2^LEC per thread),
// block pass 2^LRB points (E = 2^LEB); CC / CB columns / blocks per workgroup.
// LRC / LRB must match pass_split(), which lays out the block-major twiddles.
// ---------------------------------------------------------------------------
template <int LOGN>
struct Cfg;
template <>
struct Cfg<12> {
  static constexpr int LRC = 6, LEC = 3, LRB = 6, LEB = 3, CC = 16, CB = 16;
};
template <>
struct Cfg<16> {
  static constexpr int LRC = 8, LEC = 4, LRB = 8, LEB = 4, CC = 32, CB = 32;
};
// N = 2^17: 256-point columns as at 2^16 (two radix-16 rounds, the shape the
// fused conversion runs best with) and 512-point blocks in three radix-8
// rounds, one block per wave, 16 blocks per workgroup (64-byte runs).
template <>
struct Cfg<17> {
  static constexpr int LRC = 8, LEC = 4, LRB = 9, LEB = 3, CC = 32, CB = 16;
};

template <int LOGN>
constexpr bool split_matches() {
  return pass_split_lrc(LOGN) == Cfg<LOGN>::LRC && pass_split_lrc(LOGN) + Cfg<LOGN>::LRB == LOGN;
}
static_assert(split_matches<12>() && split_matches<16>() && split_matches<17>(),
              "kernel pass shapes must match the host twiddle layout");

template <int LOGN>
constexpr int col_threads() {
  return Cfg<LOGN>::CC << (Cfg<LOGN>::LRC - Cfg<LOGN>::LEC);
}
template <int LOGN>
constexpr int blk_threads() {
  return Cfg<LOGN>::CB << (Cfg<LOGN>::LRB - Cfg<LOGN>::LEB);
}
template <int LOGN>
constexpr int col_tiles() {
  return (1 << Cfg<LOGN>::LRB) / Cfg<LOGN>::CC;
}
static inline int col_tiles_of(uint32_t log2n) {
  return log2n == 12 ? col_tiles<12>() : log2n == 16 ? col_tiles<16>() : col_tiles<17>();
}
template <int LOGN>
constexpr int blk_tiles() {
  return (1 << Cfg<LOGN>::LRC) / Cfg<LOGN>::CB;
}

// ---------------------------------------------------------------------------
// limb policies
// ---------------------------------------------------------------------------
// Segment layout (store_tile_segments): a limb of N = 2^(lrc + lrb) words is
// 2^lrb rows of 2^lrc columns, position row 2^lrc + col; segment col holds
// column col, natural row bitrev(x) at offset col 2^lrb + x. Under X -> X^g
// the position p = row 2^lrc + col reads source position g p + h mod N, that
// is column (g col + h) mod 2^lrc, row (g row + floor((g col + h) / 2^lrc))
// mod 2^lrb: all rows of one output column come from one source column, one
// 2^lrb-word segment.
__device__ __forceinline__ uint32_t seg_src_index(uint32_t p, uint32_t g, uint32_t h, int lrc, int lrb) {
  const uint32_t cmask = (1u << lrc) - 1, rmask = (1u << lrb) - 1;
  const uint32_t u = (p & cmask) * g + h;
  const uint32_t row = ((p >> lrc) * g + (u >> lrc)) & rmask;
  return ((u & cmask) << lrb) | (__brev(row) >> (32 - lrb));
}

struct PlainLimb {
  uint32_t r, rinv;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ src;
  uint32_t* __restrict__ dst;
  __device__ __forceinline__ uint32_t load(int pos) const { return at32(src, pos); }
  __device__ __forceinline__ void store(int pos, uint32_t v) const { at32(dst, pos) = v; }
};

struct ScaledLimb {
  uint32_t r, rinv, s, sp;
  const uint32_t* __restrict__ tw;
  const uint32_t* src;
  uint32_t* dst;
  __device__ __forceinline__ uint32_t load(int pos) const { return at32(src, pos); }
  __device__ __forceinline__ void store(int pos, uint32_t v) const { at32(dst, pos) = mul_shoup(v, s, sp, r); }
};

// ModDown combine: out = (acc - v) P^-1 (+ c0 at the automorphism's source
// index). acc and c0 at the E output positions of this thread are fetched
// around the transform (fwd_blk_pass_fetch). C0 selects how c0 is read:
// kNoC0 (nothing to add), kC0Same (Galois element 1: c0 at the output
// position itself), kC0Gather (natural order, source index i g + h) and
// kC0Seg (the segment layout of a 2^LRB x 2^LRC limb: a thread's E positions
// are rows of one column, so its gathers stay in one segment). The first
// polynomial of each item adds c0, the second does not (c0 is nullptr there).
// acc (written by the inner product, read once here) and out take the
// streaming hint.
constexpr int kNoC0 = 0, kC0Same = 1, kC0Gather = 2, kC0Seg = 3;

template <int E, int LRC, int LRB, int C0>
struct CombineLimb {
  uint32_t r, rinv, pinv, pinvp;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ src;
  const uint32_t* __restrict__ acc;
  const uint32_t* __restrict__ c0;  // nullptr: nothing to add
  uint32_t g, h, mask;
  uint32_t* __restrict__ dst;
  uint32_t av[E], cv[E];
  __device__ __forceinline__ uint32_t load(int pos) const { return at32(src, pos); }
  __device__ __forceinline__ void fetch(int m, int pos) {
    av[m] = load_stream(acc, pos);
    if constexpr (C0 != kNoC0) {
      if (c0 != nullptr) {
        uint32_t si = (uint32_t)pos;
        if constexpr (C0 == kC0Gather) si = ((uint32_t)pos * g + h) & mask;
        if constexpr (C0 == kC0Seg) si = seg_src_index((uint32_t)pos, g, h, LRC, LRB);
        cv[m] = at32(c0, si);
      }
    }
  }
  __device__ __forceinline__ void finish(int m, int pos, uint32_t v) const {
    uint32_t o = mul_shoup(sub_mod(av[m], v, r), pinv, pinvp, r);
    if constexpr (C0 != kNoC0) {
      if (c0 != nullptr) o = add_mod(o, cv[m], r);
    }
    store_stream(dst, pos, o);
  }
};

// ---------------------------------------------------------------------------
// generic NTT / iNTT over a list of limbs
// ---------------------------------------------------------------------------
struct NttArgs {
  DevTables T;
  uint32_t* data;
  uint32_t* tmp;
  int N;
  uint8_t pidx[kMaxLimbsPerLaunch];
};

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_ntt_fwd_col(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  PlainLimb L{A.T.r[pi], A.T.rinv[pi], A.T.tw_fwd + pi * A.N, A.data + z * A.N, A.tmp + z * A.N};
  fwd_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_ntt_fwd_blk(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  PlainLimb L{A.T.r[pi], A.T.rinv[pi], A.T.tw_fblk + pi * A.N, A.tmp + z * A.N, A.data + z * A.N};
  fwd_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_ntt_inv_blk(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  PlainLimb L{A.T.r[pi], A.T.rinv[pi], A.T.tw_iblk + pi * A.N, A.data + z * A.N, A.tmp + z * A.N};
  inv_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_ntt_inv_col(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  ScaledLimb L{A.T.r[pi], A.T.rinv[pi], A.T.ninv[pi], A.T.ninvp[pi], A.T.tw_inv + pi * A.N,
               A.tmp + z * A.N, A.data + z * A.N};
  inv_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

// ---------------------------------------------------------------------------
// ModUp
// ---------------------------------------------------------------------------
struct ModUpArgs {
  DevTables T;
  DevLevelTables LT;
  const uint32_t* ct;  // c1 of batch item b at ct + b * ct_stride + c1_off
  uint64_t ct_stride;
  uint32_t c1_off;
  uint32_t* y;    // [batch][l][ys]
  uint32_t* tmp;  // [batch][beta][l+K][N]
  uint32_t* ext;  // [batch][beta][l+K][N]
  int N, level, K, L, alpha, beta, batch, ngroups;
  int seg;  // ext in the segment layout, the digits' own limbs included (gathers follow)
  int ys;   // words between limbs of y (N + kLimbPad)
  size_t scale_off, bconv_off;
};

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_modup_inv_blk(ModUpArgs A) {
  using C = Cfg<LOGN>;
  // rows in storage order (limb fastest): the limbs that run at the same time
  // are neighbours in memory
  const size_t b = blockIdx.y / A.level, i = blockIdx.y % A.level, z = b * A.level + i;
  PlainLimb L{A.T.r[i], A.T.rinv[i], A.T.tw_iblk + i * A.N, A.ct + b * A.ct_stride + A.c1_off + i * A.N,
              A.y + z * A.ys};
  // with the segment layout, c1's limb i is also the own limb of digit i / alpha
  uint32_t* own = A.seg ? A.ext + ((b * A.beta + i / A.alpha) * (A.level + A.K) + i) * A.N : nullptr;
  inv_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB, own);
}

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_modup_inv_col(ModUpArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, i = z % A.level;
  ScaledLimb L{A.T.r[i],          A.T.rinv[i], A.LT.mu_scale[A.scale_off + i], A.LT.mu_scalep[A.scale_off + i],
               A.T.tw_inv + i * A.N, A.y + z * A.ys, A.y + z * A.ys};
  inv_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

// XCD-aware decode of a 1-D grid of units x groups. Workgroup i runs on XCD
// i mod 8; all groups of one unit (the workgroups that read the same source
// tiles) go to the same XCD in consecutive slots, so their shared reads hit that
// XCD's L2. The grid has ceil(units / 8) * 8 * groups workgroups; padding ones
// return false.
__device__ __forceinline__ bool xcd_unit(int tiles, int rows, int groups, int& tile, int& row, int& grp) {
  const int i = (int)blockIdx.x;
  const int xcd = i & 7, slot = i >> 3;
  grp = slot % groups;
  const int unit = (slot / groups) * 8 + xcd;
  if (unit >= tiles * rows) return false;
  tile = unit % tiles;
  row = unit / tiles;
  return true;
}

static inline uint32_t xcd_grid(int tiles, int rows, int groups) {
  return (uint32_t)(((tiles * rows + 7) / 8) * 8 * groups);
}

// Grouped fast base conversion fused with the forward column pass: one
// workgroup converts G targets at once, streaming each source column tile once
// (two sources per REDC), then runs the G column passes. Source tiles are
// therefore read ceil(targets / G) times instead of once per target.
template <int G, int E>
struct TargetGroup {
  int n;          // valid targets in this group (uniform)
  int j[G];       // target limb index
  uint32_t r[G], rinv[G];
  size_t pidx[G];  // prime index of the target
  uint32_t z[G][E];
};

// r 2^32 folded out of a 64-bit sum whose high word is below 2r.
__device__ __forceinline__ uint64_t fold_hi(uint64_t x, uint32_t r) {
  uint32_t hi = (uint32_t)(x >> 32);
  hi = min(hi, hi - r);
  return ((uint64_t)hi << 32) | (uint32_t)x;
}

// sum_k v[k] c[k] 2^-32 mod r over CNT products with v[k] < 2^31 and
// c[k] < r, with one REDC: four products sum below 2r 2^32, and after each
// fold (high word below r) two more do, so the sum is folded after the fourth
// product, after every further pair and once more after an odd tail.
// The running sum is pinned to one 64-bit register pair after every step, so
// that each product is one multiply-add into it: left free, the compiler
// splits the sum into separate chains and high-word sums, which costs moves
// and 64-bit adds (18 instructions instead of 14 at CNT = 6).
template <int CNT>
__device__ __forceinline__ uint32_t dot_redc(const uint32_t (&v)[CNT], const uint32_t (&c)[CNT], uint32_t r,
                                             uint32_t rinv) {
  uint64_t acc = 0;
#pragma unroll
  for (int k = 0; k < CNT; ++k) {
    acc += mul_wide(v[k], c[k]);
    asm volatile("" : "+v"(acc));
    if (k == 3 || (k > 3 && (k & 1))) {
      acc = fold_hi(acc, r);
      asm volatile("" : "+v"(acc));
    }
  }
  constexpr bool folded_last = CNT == 4 || (CNT > 4 && !(CNT & 1));
  if constexpr (CNT > 2 && !folded_last) {
    acc = fold_hi(acc, r);
    asm volatile("" : "+v"(acc));
  }
  return redc(acc, r, rinv);
}

// Grouped conversion, a few positions at a time: the source values of MC
// positions are loaded once and dotted with each target's constants, while
// the loads of the next MC positions are in flight (compiler memory barriers
// keep it from hoisting every load and spending a register on each).
// CNT is the source count the kernel is built for; a row with cnt < CNT
// sources (the last, shorter digit) repeats its last source with constant 0.
// Slots m >= E/2 (the upper half of the column's first NTT stage) use the
// constants cstw, which carry that stage's twiddle.
template <int G, int E, int CNT, class SrcFn, class ConstFn, class ConstWFn>
__device__ __forceinline__ void grouped_bconv(TargetGroup<G, E>& tg, int cnt, SrcFn src, ConstFn cst,
                                              ConstWFn cstw) {
  constexpr int MC = 2, CHUNKS = E / MC;
  static_assert(E % MC == 0 && (E / 2) % MC == 0, "positions must tile into chunks");
  uint32_t c[G][CNT], cw[G][CNT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < CNT; ++k) {
      const uint32_t x = cst(min(k, cnt - 1), g), xw = cstw(min(k, cnt - 1), g);
      c[g][k] = k < cnt ? x : 0u;
      cw[g][k] = k < cnt ? xw : 0u;
    }
  uint32_t v[2][MC][CNT];
  auto load = [&](int chunk, uint32_t (&buf)[MC][CNT]) {
#pragma unroll
    for (int i = 0; i < MC; ++i)
#pragma unroll
      for (int k = 0; k < CNT; ++k) buf[i][k] = src(min(k, cnt - 1), chunk * MC + i);
  };
  load(0, v[0]);
#pragma unroll
  for (int ch = 0; ch < CHUNKS; ++ch) {
    if (ch + 1 < CHUNKS) load(ch + 1, v[(ch + 1) & 1]);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < MC; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        tg.z[g][ch * MC + i] = dot_redc<CNT>(v[ch & 1][i], ch * MC < E / 2 ? c[g] : cw[g], tg.r[g], tg.rinv[g]);
        asm volatile("" : "+v"(tg.z[g][ch * MC + i]));  // computed here, before the next loads
      }
    asm volatile("" ::: "memory");
  }
}

// Targets per conversion workgroup: 3, or 1 when a grid of 3-target groups
// would give the chip's 256 CUs fewer than two workgroups each (a single
// ciphertext): each source tile is then read once per target (from L2), but
// three times as many workgroups share the work.
constexpr int kBconvGroup = 3;
constexpr uint32_t kBconvSmallGrid = 512;

// ModUp conversion: row (b, d), column tile blockIdx.x, target group blockIdx.z.
template <int LOGN, int CNT, int G>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_modup_bconv(ModUpArgs A) {
  using C = Cfg<LOGN>;
  constexpr int E = 1 << C::LEC;
  __shared__ uint32_t lds[C::CC * LdsTile<C::LRC, C::LEC>::STRIDE];
  const int lk = A.level + A.K;
  int tile, row, grp;
  if (!xcd_unit(col_tiles<LOGN>(), A.batch * A.beta, A.ngroups, tile, row, grp)) return;
  const int d = row % A.beta;
  const size_t b = row / A.beta;
  const int i0 = d * A.alpha, cnt = min(A.alpha, A.level - i0);
  const int T = lk - cnt;
  const int tt0 = grp * G;
  if (tt0 >= T) return;
  const int col0 = tile * C::CC;
  TargetGroup<G, E> tg;
  tg.n = min(G, T - tt0);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int tt = tt0 + min(g, tg.n - 1);
    const int j = tt < i0 ? tt : tt + cnt;
    tg.j[g] = j;
    tg.pidx[g] = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
    tg.r[g] = A.T.r[tg.pidx[g]];
    tg.rinv[g] = A.T.rinv[tg.pidx[g]];
  }
  const uint32_t* ybase = A.y + (b * A.level + i0) * A.ys;
  const uint32_t* cbase = A.LT.mu_bconv + A.bconv_off + (size_t)i0 * lk;
  const uint32_t* cwbase = A.LT.mu_bconvw + A.bconv_off + (size_t)i0 * lk;
  grouped_bconv<G, E, CNT>(
      tg, cnt,
      [&](int k, int m) {
        const uint32_t* yk = ybase + (size_t)k * A.ys;  // uniform limb base, 32-bit offset
        return at32(yk, col_pos_fwd_in<C::LRC, C::LEC, C::LRB, C::CC>(col0, m));
      },
      [&](int k, int g) { return cbase[(size_t)k * lk + tg.j[g]]; },
      [&](int k, int g) { return cwbase[(size_t)k * lk + tg.j[g]]; });
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < tg.n) {
      fwd_col_compute<C::LRC, C::LEC, C::CC, true>(tg.z[g], lds, tg.r[g], tg.rinv[g],
                                                   A.T.tw_fwd + tg.pidx[g] * A.N);
      uint32_t* dst = A.tmp + ((b * A.beta + d) * lk + tg.j[g]) * A.N;
#pragma unroll
      // streaming stores: the block pass reads them once, and the inner
      // product's digits (the block pass's output) keep the cache
      for (int m = 0; m < E; ++m) store_stream(dst, col_pos_fwd_out<C::LRC, C::LEC, C::LRB, C::CC>(col0, m), tg.z[g][m]);
    }
  }
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_modup_fwd_blk(ModUpArgs A) {
  using C = Cfg<LOGN>;
  const int lk = A.level + A.K;
  // rows in storage order (see k_modup_inv_blk)
  const int j = (int)(blockIdx.y % lk);
  const size_t bd = blockIdx.y / lk, z = bd * lk + j;
  const int d = (int)(bd % A.beta);
  const int i0 = d * A.alpha;
  if (j >= i0 && j < min(i0 + A.alpha, A.level)) return;
  const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
  PlainLimb L{A.T.r[pj], A.T.rinv[pj], A.T.tw_fblk + pj * A.N, A.tmp + z * A.N, A.ext + z * A.N};
  // tile order rotated by the prime: neighbouring limbs, which run at the same
  // time, then touch different offsets, while each XCD still serves one tile
  // (one slice of the twiddles) per prime
  const int tile = (int)((blockIdx.x + (uint32_t)j) % (uint32_t)blk_tiles<LOGN>());
  fwd_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, tile * C::CB, A.seg != 0);
}

// ---------------------------------------------------------------------------
// inner product with the key: acc_u[j] = sum_d phi(ext_d[j]) * (b_d[j], a_d[j])
// A thread owns 8 positions of limb j for one key and loops over the batch, so
// the key values (b read, a read or regenerated) are loaded once per batch.
// The 8 positions are two runs of 4, at p0 and p1: where a thread also expands
// its own ChaCha block, p1 = p0 + 4 (the block's 8 consecutive positions);
// otherwise p1 = p0 + half a tile and consecutive lanes own consecutive
// 16-byte chunks, so every load and store instruction covers whole cache lines.
// Products are reduced with REDC in pairs; b and a are first put in
// Montgomery form, so the accumulators carry a factor 2^-64 that ModDown's
// constants remove.
// ---------------------------------------------------------------------------
struct IPArgs {
  DevTables T;
  const uint32_t* ct;
  uint64_t ct_stride;
  uint32_t c1_off;
  const uint32_t* ext;  // [batch][beta][l+K][N]
  uint32_t* acc;        // [items][2][l+K][N], item = key * batch + b
  int N, level, K, L, alpha, batch, nkeys;
  int key_level;  // level of the keys (their limbs are [q_0..q_{key_level-1}, p_0..p_{K-1}])
  int limb_xcd;   // 0, or the split of limb_xcd_decode: tiles of limb j grouped on XCDs (see below)
  int lrc, lrb;   // N = 2^(lrc + lrb): columns and rows of the segment layout
  uint32_t key_base;
  // 0: every key reads the same batch; else key k reads the ciphertext and ext
  // at these offsets (words) times k (one ciphertext per key, as in the giant
  // steps of a linear transform)
  uint64_t ct_key_stride, ext_key_stride;
  const uint32_t* evk_b[kMaxKeysPerLaunch];
  const uint32_t* evk_a[kMaxKeysPerLaunch];
  ChaChaKey seed[kMaxKeysPerLaunch];
  uint32_t galois[kMaxKeysPerLaunch];
};

__device__ __forceinline__ int pos8(int p0, int p1, int k) { return k < 4 ? p0 + k : p1 + k - 4; }

// Key-basis index of limb j of the extended basis at the ciphertext's level
// (the q limbs keep their index; the special primes follow the key's own q limbs).
__device__ __forceinline__ int key_limb(const IPArgs& A, int j) { return j < A.level ? j : A.key_level + (j - A.level); }

__device__ __forceinline__ void load8(const uint32_t* base, int p0, int p1, uint32_t (&v)[8]) {
  const uint4 x = *reinterpret_cast<const uint4*>(&at32(base, p0));
  const uint4 y = *reinterpret_cast<const uint4*>(&at32(base, p1));
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
  v[4] = y.x;
  v[5] = y.y;
  v[6] = y.z;
  v[7] = y.w;
}

__device__ __forceinline__ void store8(uint32_t* base, int p0, int p1, const uint32_t (&v)[8]) {
  *reinterpret_cast<uint4*>(&at32(base, p0)) = make_uint4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<uint4*>(&at32(base, p1)) = make_uint4(v[4], v[5], v[6], v[7]);
}

// Key values of digit d, limb j at the thread's 8 positions, in Montgomery form.
__device__ __forceinline__ void load_key8(const uint32_t* limb, int p0, int p1, uint32_t r, uint32_t rinv,
                                          uint32_t (&m)[8]) {
  uint32_t w[8];
  load8(limb, p0, p1, w);
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = redc(w[k], r, rinv);
}

// phi(ext_d[j]) of batch item b at the thread's 8 positions: the digit's own
// limbs come straight from c1, the others from ModUp's output; the automorphism
// index map is a gather unless the Galois element is 1. With the segment
// layout (SEG) every limb, own ones included, is read from ext at src_idx.
template <int BETA, bool SEG>
__device__ __forceinline__ void load_digits(const IPArgs& A, int key, int b, int j, int lk, uint32_t g, int p0, int p1,
                                            const uint32_t (&src_idx)[8], uint32_t (&e)[BETA][8]) {
  // with SEG the offsets are made opaque per call: otherwise the compiler
  // keeps a 64-bit address per digit and position live across the batch loop
  uint32_t idx[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    idx[k] = src_idx[k];
    if constexpr (SEG) asm volatile("" : "+v"(idx[k]));
  }
#pragma unroll
  for (int d = 0; d < BETA; ++d) {
    const bool own = !SEG && j < A.level && j >= d * A.alpha && j < (d + 1) * A.alpha;
    const uint32_t* src = own ? A.ct + key * A.ct_key_stride + b * A.ct_stride + A.c1_off + (size_t)j * A.N
                              : A.ext + key * A.ext_key_stride + (((size_t)b * BETA + d) * lk + j) * A.N;
    if (!SEG && g == 1u) {
      load8(src, p0, p1, e[d]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) e[d][k] = at32(src, idx[k]);
    }
  }
}

// Source index of each of the thread's 8 positions under the automorphism
// i -> i*g + (g-1)/2 mod N.
__device__ __forceinline__ void gather_index(int N, uint32_t g, int p0, int p1, uint32_t (&idx)[8]) {
  const uint32_t h = (g - 1) >> 1, mask = (uint32_t)N - 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) idx[k] = ((uint32_t)pos8(p0, p1, k) * g + h) & mask;
}

// Position of run `run` (8 consecutive positions, one ChaCha block) when runs
// walk each 8-column strip down its rows: the lanes of a wave hold consecutive
// rows of one strip, so each of a thread's 8 gathers reads, across the wave,
// a single segment.
__device__ __forceinline__ int seg_run_pos(int run, int lrc, int lrb) {
  return ((run & ((1 << lrb) - 1)) << lrc) + ((run >> lrb) << 3);
}

__device__ __forceinline__ void gather_index_seg(const IPArgs& A, uint32_t g, int p0, uint32_t (&idx)[8]) {
  const uint32_t h = (g - 1) >> 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) idx[k] = seg_src_index((uint32_t)(p0 + k), g, h, A.lrc, A.lrb);
}

// (sum_d e_d b_d, sum_d e_d a_d) at one position; am(d) gives a_d there.
// Each sum is one dot_redc: the products add up in 64 bits with folds, and a
// single REDC ends it (b and a are below r, e below 2^31).
template <int BETA, class AFn>
__device__ __forceinline__ void ip_sums(const uint32_t (&e)[BETA][8], const uint32_t (&bm)[BETA][8], int k, AFn am,
                                        uint32_t r, uint32_t rinv, uint32_t& s0, uint32_t& s1) {
  uint32_t ev[BETA], bv[BETA], av[BETA];
#pragma unroll
  for (int d = 0; d < BETA; ++d) {
    ev[d] = e[d][k];
    bv[d] = bm[d][k];
    av[d] = am(d);
  }
  s0 = dot_redc<BETA>(ev, bv, r, rinv);
  s1 = dot_redc<BETA>(ev, av, r, rinv);
}

constexpr int kIpThreads = 256;

// Placement for gathers under automorphisms: a gather reads the whole source
// limb, so the tiles of one limb (for every key or item that gathers from it)
// go to the same XCD, and each limb fills one L2 instead of all eight.
// Workgroup i of a 1-D grid runs on XCD i mod 8. With few limbs, whole limbs
// would load the 8 XCDs unevenly, so a limb can be cut into `split` parts of
// tiles/split tiles: part s of limb j is part j split + s of the walk, on XCD
// (j split + s) mod 8, and the limb fills `split` L2s. The walk has
// 8 ceil(limbs split / 8) per_limb tiles/split units; padding units return false.
__device__ __forceinline__ bool limb_xcd_decode(int u, int tiles, int split, int limbs, int per_limb, int& tile,
                                                int& limb, int& idx) {
  const int xcd = u & 7, slot = u >> 3, tps = tiles / split;
  const int t_in = slot % tps, rest = slot / tps;
  idx = rest % per_limb;
  const int part = xcd + 8 * (rest / per_limb);
  limb = part / split;
  tile = (part % split) * tps + t_in;
  return limb < limbs;
}
__device__ __forceinline__ bool limb_xcd_unit(int tiles, int split, int limbs, int per_limb, int& tile, int& limb,
                                              int& idx) {
  return limb_xcd_decode((int)blockIdx.x, tiles, split, limbs, per_limb, tile, limb, idx);
}

// One workgroup per (tile of 8*kIpThreads positions, limb, key): a grid
// (tiles, limbs, keys), or under automorphisms the 1-D walk of
// limb_xcd_decode. STORED: the a half is read; otherwise each thread expands its
// ChaCha block per digit. BT: the batch size when known at compile time (1 or
// 8), else 0. SEG: ext is in the segment layout and a tile's runs walk strips
// (seg_run_pos).
template <int BETA, int ROUNDS, bool STORED, int BT, bool SEG>
__global__ void __launch_bounds__(kIpThreads) k_inner_product(IPArgs A) {
  constexpr int TILE = 8 * kIpThreads;
  const int lk = A.level + A.K;
  int tile = (int)blockIdx.x, j = (int)blockIdx.y, key = (int)blockIdx.z;
  if (A.limb_xcd && !limb_xcd_unit(A.N / TILE, A.limb_xcd, lk, A.nkeys, tile, j, key)) return;
  const int run = tile * kIpThreads + (int)threadIdx.x;
  const int p0 = SEG ? seg_run_pos(run, A.lrc, A.lrb) : STORED ? tile * TILE + 4 * (int)threadIdx.x : run * 8;
  const int p1 = !SEG && STORED ? p0 + TILE / 2 : p0 + 4;
  const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj];
  const uint32_t g = A.galois[key];
  const int kj = key_limb(A, j);
  uint32_t src_idx[8];
  if constexpr (SEG)
    gather_index_seg(A, g, p0, src_idx);
  else
    gather_index(A.N, g, p0, p1, src_idx);

  uint32_t bm[BETA][8], am[BETA][8];
#pragma unroll
  for (int d = 0; d < BETA; ++d) {
    const size_t kofs = ((size_t)d * (A.key_level + A.K) + kj) * A.N;
    load_key8(A.evk_b[key] + kofs, p0, p1, r, rinv, bm[d]);
    if constexpr (STORED) {
      load_key8(A.evk_a[key] + kofs, p0, p1, r, rinv, am[d]);
    } else {
      uint32_t w[16];
      chacha_block<ROUNDS>(A.seed[key], (uint32_t)(p0 >> 3), 0u, (uint32_t)d, (uint32_t)kj, w);
#pragma unroll
      for (int k = 0; k < 8; ++k) am[d][k] = word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv);
    }
  }

  const int batch = BT ? BT : A.batch;
#pragma unroll 1
  for (int b = 0; b < batch; ++b) {
    uint32_t e[BETA][8];
    load_digits<BETA, SEG>(A, (int)A.key_base + key, b, j, lk, g, p0, p1, src_idx, e);
    uint32_t o0[8], o1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ip_sums<BETA>(e, bm, k, [&](int d) { return am[d][k]; }, r, rinv, o0[k], o1[k]);
    const size_t item = (size_t)(A.key_base + key) * A.batch + b;
    store8(A.acc + ((item * 2 + 0) * lk + j) * A.N, p0, p1, o0);
    store8(A.acc + ((item * 2 + 1) * lk + j) * A.N, p0, p1, o1);
  }
}

// Inner product with the a half regenerated from ChaCha, for batches of two or
// more ciphertexts. Each workgroup splits into producer waves, which expand the
// a half of the next unit (key, limb j, tile of 8*kIpHalf positions) into LDS,
// and consumer waves, which stream the current unit's digits and accumulators
// for the whole batch; the ChaCha arithmetic thus runs under the HBM traffic,
// and the consumers' layout (two runs of 4 at p0 and p0 + 4*kIpHalf) is free
// of the ChaCha block layout. Workgroups walk the units with a stride of the
// grid size; both halves expand the first unit together.
constexpr int kIpHalf = 128;  // consumer threads = producer threads per workgroup

template <int BETA, int ROUNDS, int BT, bool SEG>
__global__ void __launch_bounds__(2 * kIpHalf) k_ip_regen(IPArgs A) {
  constexpr int TILE = 8 * kIpHalf;
  __shared__ uint32_t am_lds[2][BETA][8][kIpHalf];  // [slot][digit][k][consumer thread]
  const int lk = A.level + A.K;
  const int tiles = A.N / TILE;
  // under automorphisms, units are numbered as in limb_xcd_decode, so that
  // unit u, walked by workgroup u mod gridDim.x (a multiple of 8), runs on
  // XCD u mod 8 with its limb's other tiles; the padding units are skipped
  const int units = A.limb_xcd ? 8 * ((lk * A.limb_xcd + 7) / 8) * A.nkeys * (tiles / A.limb_xcd)
                               : A.nkeys * lk * tiles;
  const bool producer = threadIdx.x >= kIpHalf;
  const int t = threadIdx.x % kIpHalf;
  int u = blockIdx.x;
  if (u >= units) return;  // uniform over the workgroup

  auto decode = [&](int unit, int& key, int& j, int& tile) {
    if (A.limb_xcd) return limb_xcd_decode(unit, tiles, A.limb_xcd, lk, A.nkeys, tile, j, key);
    tile = unit % tiles;
    j = (unit / tiles) % lk;
    key = unit / (tiles * lk);
    return true;
  };
  // a half of digits [d0, d1) of `unit`: this thread expands ChaCha block
  // tile*kIpHalf + t (tile positions 8t..8t+7) and files each value under the
  // consumer thread and slot that own its position; with SEG, consumer t owns
  // exactly the block of run tile*kIpHalf + t (seg_run_pos)
  auto produce = [&](int unit, int slot, int d0, int d1) {
    int key, j, tile;
    if (!decode(unit, key, j, tile)) return;
    const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
    const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj];
    const int hi = (8 * t) >= TILE / 2;
    const int ct0 = (8 * t - hi * (TILE / 2)) >> 2;  // consumer thread of positions 8t..8t+3
    const int run = tile * kIpHalf + t;
    const uint32_t block = SEG ? (uint32_t)(seg_run_pos(run, A.lrc, A.lrb) >> 3) : (uint32_t)run;
#pragma unroll
    for (int d = 0; d < BETA; ++d) {
      if (d < d0 || d >= d1) continue;
      uint32_t w[16];
      chacha_block<ROUNDS>(A.seed[key], block, 0u, (uint32_t)d, (uint32_t)key_limb(A, j), w);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t v = word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv);
        if constexpr (SEG)
          am_lds[slot][d][k][t] = v;
        else
          am_lds[slot][d][4 * hi + (k & 3)][ct0 + (k >> 2)] = v;
      }
      // one digit's block at a time: interleaving the digits' ChaCha states
      // would take every register
      asm volatile("" ::: "memory");
    }
  };
  auto consume = [&](int unit, int slot) {
    int key, j, tile;
    if (!decode(unit, key, j, tile)) return;
    const int p0 = SEG ? seg_run_pos(tile * kIpHalf + t, A.lrc, A.lrb) : tile * TILE + 4 * t;
    const int p1 = SEG ? p0 + 4 : p0 + TILE / 2;
    const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
    const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj];
    const uint32_t g = A.galois[key];
    uint32_t src_idx[8];
    if constexpr (SEG)
      gather_index_seg(A, g, p0, src_idx);
    else
      gather_index(A.N, g, p0, p1, src_idx);
    uint32_t bm[BETA][8];
#pragma unroll
    for (int d = 0; d < BETA; ++d)
      load_key8(A.evk_b[key] + ((size_t)d * (A.key_level + A.K) + key_limb(A, j)) * A.N, p0, p1, r, rinv, bm[d]);
    const int batch = BT ? BT : A.batch;
#pragma unroll 1
    for (int b = 0; b < batch; ++b) {
      // the a values are re-read from LDS for every item (an opaque slot index
      // keeps the compiler from hoisting 8*BETA registers out of the loop)
      int sl = slot;
      asm volatile("" : "+s"(sl));
      uint32_t e[BETA][8];
      load_digits<BETA, SEG>(A, (int)A.key_base + key, b, j, lk, g, p0, p1, src_idx, e);
      uint32_t o0[8], o1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        ip_sums<BETA>(e, bm, k, [&](int d) { return am_lds[sl][d][k][t]; }, r, rinv, o0[k], o1[k]);
      const size_t item = (size_t)(A.key_base + key) * A.batch + b;
      store8(A.acc + ((item * 2 + 0) * lk + j) * A.N, p0, p1, o0);
      store8(A.acc + ((item * 2 + 1) * lk + j) * A.N, p0, p1, o1);
    }
  };

  if (producer)
    produce(u, 0, BETA / 2, BETA);
  else
    produce(u, 0, 0, BETA / 2);
  __syncthreads();
  int slot = 0;
#pragma unroll 1
  for (; u < units; u += gridDim.x, slot ^= 1) {
    if (producer) {
      if (u + (int)gridDim.x < units) produce(u + gridDim.x, slot ^ 1, 0, BETA);
    } else {
      consume(u, slot);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// ModUp's forward block pass fused with the inner product, for one key of
// Galois element 1 (the relinearisation shape). With no automorphism the
// inner product is pointwise, and a block-pass tile of columns [c0, c0 + CF)
// covers the same positions (row bitrev(x) 2^LRC + column) for every digit and
// item. A workgroup owns one tile of one limb j of the extended basis: it puts
// the key's values at its positions on chip once (b in registers; a in
// registers for the first AREG digits and in LDS for the others, regenerated
// from ChaCha or read from the stored half), then for each batch item runs the
// block pass of every digit's column-pass output (the digit that owns j reads
// c1's limb instead), adds the products into 64-bit sums and stores only the
// two accumulators. ext is neither stored nor read back.
// ---------------------------------------------------------------------------
struct ModUpIPArgs {
  DevTables T;
  const uint32_t* ct;  // c1 of batch item b at ct + b * ct_stride + c1_off
  uint64_t ct_stride;
  uint32_t c1_off;
  const uint32_t* tmp;  // [batch][beta][l+K][N] ModUp after the column pass
  uint32_t* acc;        // [batch][2][l+K][N]
  const uint32_t* evk_b;  // [beta_key][key_level+K][N]
  const uint32_t* evk_a;  // same shape, or nullptr: regenerated from seed
  ChaChaKey seed;
  int N, level, K, L, alpha, batch, key_level;
};

// Columns per fused tile: whole ChaCha blocks (8 consecutive positions) per
// row. 256-point blocks of 16 words per thread (N = 2^16) take 16 columns, so
// that the key's, c1's and the outputs' runs are 64 bytes long (measured per
// batch-8 launch: 8 columns 150 us, 16 columns 139 us, 32 columns 154 us with
// 16 CUs idle, and with the block pass's own order, 16-byte runs, 227 us);
// other shapes take 8.
template <int LOGN>
constexpr int fused_cols() {
  return (Cfg<LOGN>::LRB == 8 && Cfg<LOGN>::LEB == 4) ? 16 : 8;
}
// Key values a thread keeps per half (beta digits x its E positions): larger
// shapes take the separate block pass and inner product.
constexpr int kFusedKeyValues = 64;

template <int LOGN>
constexpr int fused_threads() {
  return fused_cols<LOGN>() << (Cfg<LOGN>::LRB - Cfg<LOGN>::LEB);
}
// a-half digits kept in registers (the rest sit in LDS), and the waves per
// SIMD the register budget is cut for: at N = 2^16 a 4-digit tile in 256
// threads then takes 81 KB of LDS (two a digits, the double-buffered exchange
// tile and the twiddles) and at most 256 registers, so that two workgroups
// share a CU and the 480 tiles of 30 limbs run in one wave of workgroups
template <int LOGN, int BETA>
constexpr int fused_areg() {
  return LOGN == 16 ? (BETA < 2 ? BETA : 2) : LOGN == 17 ? (BETA < 3 ? BETA : 3) : 0;
}
template <int LOGN>
constexpr int fused_waves() {
  return 2;
}

// LDS layout of a fused tile of C blocks (8 or 16): the block pass's padded
// rows, col(x) = x + x/16 at N = 2^16, with row(k) = 272 k + (32/C)(k >> 1).
// The exchange's two patterns put the blocks k, k + 1 of a half-wave 16 banks
// apart, as in the pass's own layout, and the transposed read of x = rest +
// 16 m across the C blocks (32/C rests per half-wave) starts the blocks on the
// C distinct multiples of 32/C, so every access covers 32 distinct banks (the
// pass's own skew, k/2, is made for 32 blocks). Other shapes keep the pass's
// layout.
template <int LRB, int LEB, int C>
struct FusedLay : BlkLds<LRB, LEB> {
  using Base = BlkLds<LRB, LEB>;
  static constexpr bool SK = Base::SWZ;
  static constexpr int SKEW = 32 / C;
  static_assert(!SK || C == 8 || C == 16, "skew made for 8 or 16 blocks");
  __device__ __forceinline__ static int row(int k) { return SK ? k * Base::S + SKEW * (k >> 1) : Base::row(k); }
  static constexpr int words(int c) { return SK ? c * Base::S + SKEW * ((c - 1) >> 1) : Base::words(c); }
};

// Tile groups: the 128 / (4 CF) tiles that share each row's 128-byte line run
// on one XCD in consecutive slots (xcd_unit with that many groups), so the
// runs of their loads and stores meet in that XCD's L2.
template <int LOGN, int BETA, int ROUNDS, bool STORED>
__global__ void __launch_bounds__(fused_threads<LOGN>(), fused_waves<LOGN>()) k_modup_ip(ModUpIPArgs A) {
  using C = Cfg<LOGN>;
  constexpr int LRC = C::LRC, LRB = C::LRB, LEB = C::LEB, CF = fused_cols<LOGN>();
  constexpr int G = 32 / CF, CB = CF / 8;  // tiles per 128-byte line, ChaCha blocks per tile row
  constexpr int E = 1 << LEB, TPB = 1 << (LRB - LEB), THREADS = CF * TPB, RB = LRB / LEB;
  constexpr int AREG = fused_areg<LOGN, BETA>(), NS = BETA - AREG > 0 ? BETA - AREG : 1;
  static_assert(CF % 8 == 0 && 32 % CF == 0, "a tile row is whole ChaCha blocks within a 128-byte line");
  static_assert(((1 << LRC) / CF) % G == 0, "tiles group by line");
  using Lay = FusedLay<LRB, LEB, CF>;
  // with TWL the exchange/transpose tile is double-buffered (NB = 2): steps
  // that run the block pass alternate between the buffers, so a step needs one
  // barrier, between its transposed write and read (a wave that reaches the
  // next step's barrier has finished this step's reads)
  constexpr int NB = LRB == 8 && LEB == 4 ? 2 : 1;
  constexpr int TW = Lay::words(CF);
  __shared__ uint32_t lds[NB * TW];
  __shared__ uint32_t am_lds[NS][E][THREADS];  // [digit - AREG][slot][consumer thread]
  // 256-point blocks of 16 words per thread (N = 2^16): the tile's twiddles
  // sit on chip for the whole batch (TWW words per block in twl, the rest in
  // registers), so the loop reads them with short LDS latency and its only
  // global loads are the inputs that are prefetched a step ahead
  constexpr bool TWL = LRB == 8 && LEB == 4;
  constexpr int TWW = 16 + 64 + 128;
  __shared__ __align__(16) uint32_t twl[TWL ? CF * TWW : 4];
  const int tid = (int)threadIdx.x;
  const int lk = A.level + A.K;
  int line, j, g;
  if (!xcd_unit((1 << LRC) / CF / G, lk, G, line, j, g)) return;
  const int c0 = (line * G + g) * CF;
  // consumer layout (after the block pass's transpose): column c0 + kk, rows
  // bitrev(rest + TPB m). rest fills the low LRB - LEB bits and TPB m the top
  // LEB, so position m = pos0 + (bitrev(m, LEB) << LRC): one per-lane offset,
  // and the constant goes into the uniform base (slot_of).
  const int kk = tid % CF, rest = tid / CF;
  const uint32_t pos0 = (bitrev((uint32_t)rest, LRB) << LRC) + (uint32_t)(c0 + kk);
  auto slot_of = [](int m) { return (size_t)bitrev((uint32_t)m, LEB) << LRC; };
  const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj];
  const int kj = j < A.level ? j : A.key_level + (j - A.level);
  const size_t kdig = (size_t)(A.key_level + A.K) * A.N;  // words per digit of the key

  // twl, block kb of the tile (natural block bitrev(c0 + kb)): words 0..14 are
  // round 0's entries 1..15 (one run shared by the block's 16 threads, word 15
  // a pad), words 16 + 4t .. 19 + 4t stage 2 of round 1 (entries 64 + 4t ..),
  // and words 80 + 64u + 4t .. 83 + 64u + 4t stage 3 of round 1 (entries
  // 128 + 8t + 4u ..), so that 8 consecutive threads' 16-byte reads cover 32
  // banks. Stages 0 and 1 of round 1 (3 entries per thread) stay in registers.
  // Thread tid fetches words tid + THREADS i; they are stored after the a half
  // is expanded, so that the fetches run under the expansion.
  constexpr int TWN = TWL ? (CF * TWW + THREADS - 1) / THREADS : 1;
  uint32_t twv[TWN];
  if constexpr (TWL) {
    const uint32_t* twp = A.T.tw_fblk + pj * A.N;
#pragma unroll
    for (int i = 0; i < TWN; ++i) {
      const int w = tid + THREADS * i;
      const int kb = w / TWW, o = w % TWW;
      const uint32_t Bk = bitrev((uint32_t)(c0 + (w < CF * TWW ? kb : 0)), LRC);
      int ent;
      if (o < 16)
        ent = o < 15 ? 1 + o : 1;
      else if (o < 80)
        ent = 64 + (o - 16);
      else {
        const int q = o - 80;
        ent = 128 + 8 * ((q % 64) / 4) + 4 * (q / 64) + (q % 4);
      }
      twv[i] = twp[(Bk << LRB) + (uint32_t)ent];
    }
  }

  // b's raw words (reduced once the a half is on chip) and the first step's
  // inputs: fetched before the a half is expanded where the registers allow
  // (EARLY), so that they arrive under the expansion; otherwise after it
  constexpr bool EARLY = TWL && !STORED;
  uint32_t bm[BETA][E];
  auto fetch_b = [&]() {
#pragma unroll
    for (int d = 0; d < BETA; ++d)
#pragma unroll
      for (int m = 0; m < E; ++m) bm[d][m] = at32(A.evk_b + d * kdig + (size_t)kj * A.N + slot_of(m), pos0);
  };

  // block-pass layout: block k of the tile, thread t within it; the round-0
  // input of slot m is word blk0 + TPB m of the limb
  const int t = tid % TPB, k = tid / TPB;
  const int B = (int)bitrev((uint32_t)(c0 + k), LRC);
  const uint32_t blk0 = ((uint32_t)B << LRB) + (uint32_t)t;
  // the block's twiddles are the same for every digit and item; shapes other
  // than TWL re-read them per round from L1 (held across the batch loop they
  // would take 2^LEB - 1 registers per round)
  const uint32_t* const tw = A.T.tw_fblk + pj * A.N;
  auto twb = [B](int st) { return (B << LRB) + (1 << st); };  // block-major table
  uint32_t w10 = 0, w11a = 0, w11b = 0;  // round 1, stages 0 and 1 (twl layout)
  if constexpr (TWL) {
    w10 = tw[twb(4) + t];
    w11a = tw[twb(5) + 2 * t];
    w11b = tw[twb(5) + 2 * t + 1];
  }
  const uint32_t* const tblk = twl + (TWL ? k * TWW : 0);
  auto lds_round_tw = [&](int rd, uint32_t (&W)[E - 1]) {
    auto q4 = [](const uint32_t* p, uint32_t* w) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x;
      w[1] = x.y;
      w[2] = x.z;
      w[3] = x.w;
    };
    if (rd == 0) {
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) q4(tblk + 4 * i, w + 4 * i);
#pragma unroll
      for (int i = 0; i < E - 1; ++i) W[i] = w[i];
    } else {
      W[0] = w10;
      W[1] = w11a;
      W[2] = w11b;
      q4(tblk + 16 + 4 * t, W + 3);
      q4(tblk + 80 + 4 * t, W + 7);
      q4(tblk + 144 + 4 * t, W + 11);
    }
  };
  uint32_t* const lrow0 = lds + Lay::row(k);
  // the transposed tile: slot m of this thread at row(kk) + col(rest) + m col(TPB)
  // (col(x) adds x/16 or x/8, and TPB is a multiple of that divisor)
  const uint32_t* const tcol0 = lds + Lay::row(kk) + Lay::col(rest);
  int buf = 0;  // the buffer of the next step that runs the block pass
  constexpr int TSTEP = (1 << LRB) / E == TPB ? TPB + (Lay::SWZ ? TPB / 16 : Lay::SWZ9 ? TPB / 8 : 0) : 0;
  static_assert(TSTEP > 0, "transposed slot stride");
  const int own_d = j < A.level ? j / A.alpha : -1;  // the digit whose own limb is j
  constexpr bool folded_last = BETA == 4 || (BETA > 4 && !(BETA & 1));
  // the next digit's inputs are loaded one step ahead, into en: c1's limb j at
  // the consumer positions for the digit that owns j, else the column-pass
  // output at the block pass's round-0 positions. With the twiddles on chip
  // they are issued at the top of the step before; otherwise after that
  // step's last twiddle loads, so that waiting for those twiddles (the counter
  // of outstanding loads is in order) never waits for them.
  // With TWL both patterns are one uniform base, one per-lane offset and a
  // uniform step per slot, selected without a branch: straight-line loads keep
  // the compiler's wait counts exact, so that they stay in flight. The other
  // shapes branch, which takes fewer registers.
  auto issue = [&](int bn, int dn, uint32_t (&x)[E]) {
    const bool own = dn == own_d;
    if constexpr (TWL) {
      const uint32_t* base = own ? A.ct + bn * A.ct_stride + A.c1_off + (size_t)j * A.N
                                 : A.tmp + (((size_t)bn * BETA + dn) * lk + j) * A.N;
      const uint32_t lane = own ? pos0 : blk0;
#pragma unroll
      for (int m = 0; m < E; ++m) x[m] = at32(base, lane + (own ? (uint32_t)slot_of(m) : (uint32_t)(TPB * m)));
    } else if (own) {
      const uint32_t* c1 = A.ct + bn * A.ct_stride + A.c1_off + (size_t)j * A.N;
#pragma unroll
      for (int m = 0; m < E; ++m) x[m] = at32(c1 + slot_of(m), pos0);
    } else {
      const uint32_t* src = A.tmp + (((size_t)bn * BETA + dn) * lk + j) * A.N;
#pragma unroll
      for (int m = 0; m < E; ++m) x[m] = at32(src, blk0 + (uint32_t)(TPB * m));
    }
  };
  uint32_t en[E];
  if constexpr (EARLY) {
    fetch_b();
    issue(0, 0, en);
    // keeps the compiler from sinking these fetches below the expansion
    asm volatile("" ::: "memory");
  }

  uint32_t am[AREG > 0 ? AREG : 1][E];
  if constexpr (STORED) {
#pragma unroll
    for (int d = 0; d < BETA; ++d)
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const uint32_t v = redc(at32(A.evk_a + d * kdig + (size_t)kj * A.N + slot_of(m), pos0), r, rinv);
        if (d < AREG)
          am[d < AREG ? d : 0][m] = v;
        else
          am_lds[d < AREG ? 0 : d - AREG][m][tid] = v;  // read back by this thread only
      }
  } else {
    // row x of the tile (natural row bitrev(x)) is CB ChaCha blocks per digit;
    // thread i expands units u = i + THREADS s (row u / CB, block h = u mod CB)
    // and files value k under consumer thread (x mod TPB) CF + 8 h + k, slot
    // x / TPB
    auto fill = [&](int d, int slot) {
#pragma unroll
      for (int s = 0; s < ((1 << LRB) * CB + THREADS - 1) / THREADS; ++s) {
        const int u = tid + THREADS * s;
        if (u >= (1 << LRB) * CB) break;
        const int x = u / CB, h = u % CB;
        const int p = (int)(bitrev((uint32_t)x, LRB) << LRC) + c0 + 8 * h;
        uint32_t w[16];
        chacha_block<ROUNDS>(A.seed, (uint32_t)(p >> 3), 0u, (uint32_t)d, (uint32_t)kj, w);
        uint32_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv);
        uint4* dst = reinterpret_cast<uint4*>(&am_lds[slot][x / TPB][(x % TPB) * CF + 8 * h]);
        dst[0] = make_uint4(v[0], v[1], v[2], v[3]);
        dst[1] = make_uint4(v[4], v[5], v[6], v[7]);
        // one block at a time: interleaved ChaCha states would take every register
        asm volatile("" ::: "memory");
      }
    };
#pragma unroll
    for (int d = 0; d < AREG; ++d) {
      fill(d, 0);
      __syncthreads();
#pragma unroll
      for (int m = 0; m < E; ++m) am[d][m] = am_lds[0][m][tid];
      __syncthreads();
    }
#pragma unroll
    for (int d = AREG; d < BETA; ++d) fill(d, d - AREG);
    __syncthreads();
  }
  // the a half is on chip: store the twiddle words and reduce b
  if constexpr (!EARLY) {
    asm volatile("" ::: "memory");
    fetch_b();
    issue(0, 0, en);
  }
  if constexpr (TWL) {
#pragma unroll
    for (int i = 0; i < TWN; ++i) {
      const int w = tid + THREADS * i;
      if (w < CF * TWW) twl[w] = twv[i];
    }
    __syncthreads();
  }
#pragma unroll
  for (int d = 0; d < BETA; ++d)
#pragma unroll
    for (int m = 0; m < E; ++m) bm[d][m] = redc(bm[d][m], r, rinv);
#pragma unroll 1
  for (int b = 0; b < A.batch; ++b) {
    // the a values in LDS are re-read for every item (an opaque base keeps the
    // compiler from hoisting them into registers across the batch loop)
    int am_base = tid;
    asm volatile("" : "+v"(am_base));
    uint64_t s0[E], s1[E];
#pragma unroll
    for (int d = 0; d < BETA; ++d) {
      const int bn = d + 1 < BETA ? b : b + 1, dn = d + 1 < BETA ? d + 1 : 0;
      uint32_t e[E];
#pragma unroll
      for (int m = 0; m < E; ++m) e[m] = en[m];
      if (d == own_d || TWL) {
        if (bn < A.batch) issue(bn, dn, en);
        // keeps the compiler from sinking the loads towards their use
        asm volatile("" ::: "memory");
      }
      if (d != own_d) {
        uint32_t* const lrow = lrow0 + (NB == 2 ? buf * TW : 0);
        const uint32_t* const tcol = tcol0 + (NB == 2 ? buf * TW : 0);
        int zero = 0;
        asm volatile("" : "+s"(zero));  // keeps the twiddle loads in the loop
#pragma unroll
        for (int rd = 0; rd < RB; ++rd) {
          uint32_t W[E - 1];
          if constexpr (TWL)
            lds_round_tw(rd, W);
          else
            load_round_tw<LRB, LEB, false>(rd, t, tw + zero, twb, W);
          if (!TWL && rd == RB - 1 && bn < A.batch) issue(bn, dn, en);
          if (rd > 0) exchange<LRB, LEB, false, Lay, block_in_wave<LRB, LEB>()>(e, lrow, rd - 1, t);
          ct_round_w<LEB>(e, W, r, rinv);
        }
#pragma unroll
        for (int m = 0; m < E; ++m) lrow[Lay::col(elem_index<LRB, LEB, false>(RB - 1, t, m))] = e[m];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < E; ++m) e[m] = tcol[TSTEP * m];
        if constexpr (NB == 1) __syncthreads();
        buf ^= 1;
      }
      // the sums of dot_redc, one digit at a time: products below r 2^31, a
      // fold after the fourth and after every further pair
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const uint32_t av = d < AREG ? am[d < AREG ? d : 0][m] : (&am_lds[d < AREG ? 0 : d - AREG][m][0])[am_base];
        if (d == 0) {
          s0[m] = mul_wide_op(e[m], bm[d][m]);
          s1[m] = mul_wide_op(e[m], av);
        } else {
          mac_wide_op(s0[m], e[m], bm[d][m]);
          mac_wide_op(s1[m], e[m], av);
        }
        if (d == 3 || (d > 3 && (d & 1))) {
          s0[m] = fold_hi(s0[m], r);
          s1[m] = fold_hi(s1[m], r);
        }
      }
    }
    uint32_t* a0 = A.acc + (((size_t)b * 2 + 0) * lk + j) * A.N;
    uint32_t* a1 = A.acc + (((size_t)b * 2 + 1) * lk + j) * A.N;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      if constexpr (BETA > 2 && !folded_last) {
        s0[m] = fold_hi(s0[m], r);
        s1[m] = fold_hi(s1[m], r);
      }
      at32(a0 + slot_of(m), pos0) = redc(s0[m], r, rinv);
      at32(a1 + slot_of(m), pos0) = redc(s1[m], r, rinv);
    }
  }
}

// ---------------------------------------------------------------------------
// ModDown
// ---------------------------------------------------------------------------
struct ModDownArgs {
  DevTables T;
  DevLevelTables LT;
  const uint32_t* acc;  // [items][polys][l+K][N]
  uint32_t* y2;         // [items][polys][K][y2s]
  uint32_t* tmp2;       // [items][polys][l][N]
  uint32_t* out;        // [items][polys][l][N]
  const uint32_t* c0;   // c0 of ciphertext b at c0 + b * ct_stride, or nullptr
  uint64_t ct_stride;
  int N, level, K, L, polys, variant, batch, rows_ip, ngroups;
  int limb_xcd;  // combine pass: 0, or the split of limb_xcd_decode (c0 gathered under an automorphism)
  int i0, ni;    // combine pass: limbs i0 .. i0 + ni - 1 of every polynomial (0 and level: all)
  int y2s;       // words between limbs of y2 (N + kLimbPad)
  uint32_t galois[kMaxKeysPerLaunch];  // per key = item / batch
};

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_md_inv_blk(ModDownArgs A) {
  using C = Cfg<LOGN>;
  const int lk = A.level + A.K;
  // rows in storage order (see k_modup_inv_blk)
  const size_t ip = blockIdx.y / A.K, t = blockIdx.y % A.K, z = ip * A.K + t, pt = A.L + t;
  PlainLimb L{A.T.r[pt], A.T.rinv[pt], A.T.tw_iblk + pt * A.N, A.acc + (ip * lk + A.level + t) * A.N,
              A.y2 + z * A.y2s};
  inv_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_md_inv_col(ModDownArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, t = z % A.K, pt = A.L + t;
  const size_t si = (size_t)A.variant * A.K + t;
  ScaledLimb L{A.T.r[pt], A.T.rinv[pt], A.LT.md_scale[si], A.LT.md_scalep[si], A.T.tw_inv + pt * A.N,
               A.y2 + z * A.y2s, A.y2 + z * A.y2s};
  inv_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

// ModDown conversion P -> q_i: row ip = (item, u), column tile blockIdx.x,
// group of G target limbs q_i blockIdx.z.
template <int LOGN, int CNT, int G>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_md_bconv(ModDownArgs A) {
  using C = Cfg<LOGN>;
  constexpr int E = 1 << C::LEC;
  __shared__ uint32_t lds[C::CC * LdsTile<C::LRC, C::LEC>::STRIDE];
  int tile, row, grp;
  if (!xcd_unit(col_tiles<LOGN>(), A.rows_ip, A.ngroups, tile, row, grp)) return;
  const size_t ip = row;
  const int tt0 = grp * G;
  if (tt0 >= A.level) return;
  const int col0 = tile * C::CC;
  TargetGroup<G, E> tg;
  tg.n = min(G, A.level - tt0);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int i = tt0 + min(g, tg.n - 1);
    tg.j[g] = i;
    tg.pidx[g] = (size_t)i;
    tg.r[g] = A.T.r[i];
    tg.rinv[g] = A.T.rinv[i];
  }
  const uint32_t* ybase = A.y2 + ip * A.K * A.y2s;
  const uint32_t* cbase = A.LT.md_bconv + (size_t)A.variant * A.K * A.L;
  const uint32_t* cwbase = A.LT.md_bconvw + (size_t)A.variant * A.K * A.L;
  grouped_bconv<G, E, CNT>(
      tg, A.K,
      [&](int k, int m) {
        const uint32_t* yk = ybase + (size_t)k * A.y2s;  // uniform limb base, 32-bit offset
        return at32(yk, col_pos_fwd_in<C::LRC, C::LEC, C::LRB, C::CC>(col0, m));
      },
      [&](int k, int g) { return cbase[(size_t)k * A.L + tg.j[g]]; },
      [&](int k, int g) { return cwbase[(size_t)k * A.L + tg.j[g]]; });
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < tg.n) {
      fwd_col_compute<C::LRC, C::LEC, C::CC, true>(tg.z[g], lds, tg.r[g], tg.rinv[g],
                                                   A.T.tw_fwd + tg.pidx[g] * A.N);
      uint32_t* dst = A.tmp2 + (ip * A.level + tg.j[g]) * A.N;
#pragma unroll
      for (int m = 0; m < E; ++m) at32(dst, col_pos_fwd_out<C::LRC, C::LEC, C::LRB, C::CC>(col0, m)) = tg.z[g][m];
    }
  }
}

// C0: how c0 is read (CombineLimb). EARLY: side inputs fetched before the
// transform (fwd_blk_pass_fetch).
template <int LOGN, int C0, bool EARLY>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_md_fwd_blk(ModDownArgs A) {
  using C = Cfg<LOGN>;
  const int lk = A.level + A.K;
  // rows in storage order (see k_modup_inv_blk); when c0 is gathered under an
  // automorphism, the tiles of limb i are grouped on XCDs (see limb_xcd_decode)
  int tile = (int)blockIdx.x, ipi = (int)(blockIdx.y / A.ni), ii = A.i0 + (int)(blockIdx.y % A.ni);
  if (A.limb_xcd && !limb_xcd_unit(blk_tiles<LOGN>(), A.limb_xcd, A.level, A.rows_ip, tile, ii, ipi)) return;
  const size_t ip = (size_t)ipi, i = (size_t)ii, z = ip * A.level + i;
  const size_t item = ip / A.polys, u = ip % A.polys;
  const size_t pi = (size_t)A.variant * A.L + i;
  const uint32_t* c0 = nullptr;
  uint32_t g = 1;
  if (A.c0 != nullptr && u == 0) {
    c0 = A.c0 + (item % A.batch) * A.ct_stride + i * A.N;
    g = A.galois[item / A.batch];
  }
  CombineLimb<(1 << C::LEB), C::LRC, C::LRB, C0> L{A.T.r[i],
                A.T.rinv[i],
                A.LT.md_pinv[pi],
                A.LT.md_pinvp[pi],
                A.T.tw_fblk + i * A.N,
                A.tmp2 + z * A.N,
                A.acc + (ip * lk + i) * A.N,
                c0,
                g,
                (g - 1) >> 1,
                (uint32_t)A.N - 1,
                A.out + z * A.N,
                {},
                {}};
  fwd_blk_pass_fetch<C::LRC, C::LRB, C::LEB, C::CB, EARLY>(L, tile * C::CB);
}

// Natural order -> segment layout, one limb per row of the grid.
struct SegCopyArgs {
  const uint32_t* src;
  uint32_t* dst;
  int N;
};

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_seg_copy(SegCopyArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y;
  copy_tile_segments<C::LRC, C::LRB, C::LEB, C::CB>(A.src + z * A.N, A.dst + z * A.N, blockIdx.x * C::CB);
}

// ---------------------------------------------------------------------------
// ChaCha expansion of one limb of the a half (debug / parity entry point)
// ---------------------------------------------------------------------------
template <int ROUNDS>
__global__ void __launch_bounds__(256) k_chacha_expand(ChaChaKey key, uint32_t d, uint32_t j, uint32_t r,
                                                       uint32_t rinv, uint32_t r2, uint32_t* dst, int N) {
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= N) return;
  uint32_t w[16];
  chacha_block<ROUNDS>(key, (uint32_t)(i0 >> 3), 0u, d, j, w);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t m = word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv);  // a 2^-32
    dst[i0 + k] = redc(mul_wide(m, r2), r, rinv);                            // a 2^-32 2^64 2^-32 = a
  }
}

// Every limb of a key's a half: grid (N / 2048, kl + K, beta), one ChaCha block
// (8 positions) per thread; limb j of the key basis at key level kl.
struct ExpandKeyArgs {
  DevTables T;
  ChaChaKey key;
  uint32_t* dst;  // [beta][kl+K][N]
  int N, kl, L;
};

template <int ROUNDS>
__global__ void __launch_bounds__(256) k_expand_key(ExpandKeyArgs A) {
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= A.N) return;
  const int j = blockIdx.y, d = blockIdx.z, lk = gridDim.y;
  const size_t pj = j < A.kl ? (size_t)j : (size_t)(A.L + j - A.kl);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj], r2 = A.T.r2[pj];
  uint32_t w[16];
  chacha_block<ROUNDS>(A.key, (uint32_t)(i0 >> 3), 0u, (uint32_t)d, (uint32_t)j, w);
  uint32_t v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = redc(mul_wide(word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv), r2), r, rinv);
  uint32_t* out = A.dst + ((size_t)d * lk + j) * A.N + i0;
  *reinterpret_cast<uint4*>(out) = make_uint4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<uint4*>(out + 4) = make_uint4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------------------
// homomorphic multiplication around the key switch
// ---------------------------------------------------------------------------
// Tensor product of ciphertext pairs: d0 = a0 b0, d1 = a0 b1 + a1 b0,
// d2 = a1 b1 per limb i = blockIdx.y, pair blockIdx.z. b is put in Montgomery
// form (b 2^32) so that each product, or the sum of the two cross products,
// is one REDC. Positions as in the inner product (two runs of 4 per thread).
struct TensorArgs {
  DevTables T;
  const uint32_t* a;  // pair z: a0 at a + z*a_stride, a1 at + l*N
  const uint32_t* b;
  uint64_t a_stride, b_stride;
  uint32_t* d;  // pair z: d_k at d + z*d_stride + d_off[k]
  uint64_t d_stride;
  uint64_t d_off[3];
  int N, level;
};

constexpr int kTensorThreads = 256;

#if PC_IN_PART(5)
__global__ void __launch_bounds__(kTensorThreads) k_tensor(TensorArgs A) {
  constexpr int TILE = 8 * kTensorThreads;
  const int i = blockIdx.y;
  const size_t z = blockIdx.z, ln = (size_t)A.level * A.N;
  const int p0 = (int)blockIdx.x * TILE + 4 * (int)threadIdx.x, p1 = p0 + TILE / 2;
  const uint32_t r = A.T.r[i], rinv = A.T.rinv[i], r2 = A.T.r2[i];
  const uint32_t* a0p = A.a + z * A.a_stride + (size_t)i * A.N;
  const uint32_t* b0p = A.b + z * A.b_stride + (size_t)i * A.N;
  uint32_t a0[8], a1[8], b0[8], b1[8];
  load8(a0p, p0, p1, a0);
  load8(a0p + ln, p0, p1, a1);
  load8(b0p, p0, p1, b0);
  load8(b0p + ln, p0, p1, b1);
  uint32_t d0[8], d1[8], d2[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t b0m = redc(mul_wide(b0[k], r2), r, rinv), b1m = redc(mul_wide(b1[k], r2), r, rinv);
    d0[k] = redc(mul_wide(a0[k], b0m), r, rinv);
    d1[k] = redc(mul_wide(a0[k], b1m) + mul_wide(a1[k], b0m), r, rinv);
    d2[k] = redc(mul_wide(a1[k], b1m), r, rinv);
  }
  uint32_t* dz = A.d + z * A.d_stride + (size_t)i * A.N;
  store8(dz + A.d_off[0], p0, p1, d0);
  store8(dz + A.d_off[1], p0, p1, d1);
  store8(dz + A.d_off[2], p0, p1, d2);
}
#endif

// Rescale by the last prime q_l' (l' = level - 1) of 2*batch polynomials:
// out_i = (c_i - NTT_i([x]_{q_l'} mod q_i)) q_l'^-1 mod q_i for i < l', with x
// the coefficients of limb l' (already inverse-transformed) and [x] its
// centred residue. The column pass loads [x] mod q_i, the block pass fetches
// c_i (plus an optional addend on the second polynomial) at its output
// positions and stores the division.
struct RescaleArgs {
  DevTables T;
  const uint32_t* x;  // [polys][N] limb l' of every polynomial, coefficient form
  const uint32_t* c;  // polynomial u = 2b + v at c + b*c_stride + v*c1_off, limb i at + i*N
  uint64_t c_stride;
  uint32_t c1_off;
  const uint32_t* add1;  // nullptr, or added to polynomial 2b+1: limb i at add1 + b*add_stride + i*N
  uint64_t add_stride;
  uint32_t* x_out;  // gather target (= x)
  uint32_t* tmp;    // [polys][l'][N]
  uint32_t* out;    // [batch][2][l'][N]
  int N, lp;        // lp = l' = level - 1
  uint32_t ql_half;
  uint32_t ql_mod[kMaxRescaleLimbs], inv[kMaxRescaleLimbs], invp[kMaxRescaleLimbs];
};

// x[u] = limb l' of polynomial u (plus the addend's limb l' on odd u).
constexpr int kGatherThreads = 256;

#if PC_IN_PART(5)
__global__ void __launch_bounds__(kGatherThreads) k_rs_gather(RescaleArgs A) {
  const size_t u = blockIdx.y, b = u >> 1, v = u & 1;
  const int pos = 4 * ((int)blockIdx.x * kGatherThreads + (int)threadIdx.x);
  const uint32_t* src = A.c + b * A.c_stride + v * A.c1_off + (size_t)A.lp * A.N;
  uint4 w = *reinterpret_cast<const uint4*>(src + pos);
  if (v == 1 && A.add1 != nullptr) {
    const uint32_t q = A.T.r[A.lp];
    const uint4 d = *reinterpret_cast<const uint4*>(A.add1 + b * A.add_stride + (size_t)A.lp * A.N + pos);
    w.x = add_mod(w.x, d.x, q);
    w.y = add_mod(w.y, d.y, q);
    w.z = add_mod(w.z, d.z, q);
    w.w = add_mod(w.w, d.w, q);
  }
  *reinterpret_cast<uint4*>(A.x_out + u * A.N + pos) = w;
}
#endif

struct RescaleSrcLimb {
  uint32_t r, rinv;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ x;
  uint32_t ql_half, ql_mod;
  uint32_t* __restrict__ dst;
  __device__ __forceinline__ uint32_t load(int pos) const {
    const uint32_t v = at32(x, pos);
    const uint32_t m = reduce_2r(v, r);  // v < 2^31 < 2r
    return v > ql_half ? sub_mod(m, ql_mod, r) : m;
  }
  __device__ __forceinline__ void store(int pos, uint32_t v) const { at32(dst, pos) = v; }
};

template <int E>
struct RescaleOutLimb {
  uint32_t r, rinv, inv, invp;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ src;
  const uint32_t* __restrict__ c;
  const uint32_t* __restrict__ add;  // nullptr: nothing to add
  uint32_t* __restrict__ dst;
  uint32_t cv[E];
  __device__ __forceinline__ uint32_t load(int pos) const { return at32(src, pos); }
  __device__ __forceinline__ void fetch(int m, int pos) {
    cv[m] = at32(c, pos);
    if (add) cv[m] = add_mod(cv[m], at32(add, pos), r);
  }
  __device__ __forceinline__ void finish(int m, int pos, uint32_t v) const {
    at32(dst, pos) = mul_shoup(sub_mod(cv[m], v, r), inv, invp, r);
  }
};

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_rs_col(RescaleArgs A) {
  using C = Cfg<LOGN>;
  const int u = blockIdx.y / A.lp, i = blockIdx.y % A.lp;
  RescaleSrcLimb L{A.T.r[i],      A.T.rinv[i], A.T.tw_fwd + (size_t)i * A.N, A.x + (size_t)u * A.N,
                   A.ql_half,     A.ql_mod[i], A.tmp + ((size_t)u * A.lp + i) * A.N};
  fwd_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

// The ModDown combine of a relinearisation (as k_md_fwd_blk with Galois
// element 1) and the rescale's last pass (as k_rs_blk) for limb i < l' of
// polynomial u, in one workgroup: two block passes on the same prime and
// tile, the relinearised value o kept in registers between them instead of
// being written and read back.
//   phase 0: o = (acc - v) P^-1 (+ d0 on u = 0)
//   phase 1: out = (o (+ d1 on u = 1) - v) q_{l'}^-1
// acc and out take the streaming hint, as in the ModDown combine.
template <int E>
struct MdRsLimb {
  uint32_t r, rinv;
  const uint32_t* __restrict__ tw;
  uint32_t pinv, pinvp, inv, invp;
  const uint32_t* __restrict__ src_md;  // ModDown conversion, after its column pass
  const uint32_t* __restrict__ src_rs;  // rescale column-pass output
  const uint32_t* __restrict__ acc;
  const uint32_t* __restrict__ c0;   // nullptr: nothing to add
  const uint32_t* __restrict__ add;  // nullptr: nothing to add
  uint32_t* __restrict__ dst;
  int phase;
  uint32_t av[E], cv[E], o[E];
  __device__ __forceinline__ uint32_t load(int pos) const { return at32(phase ? src_rs : src_md, pos); }
  __device__ __forceinline__ void fetch(int m, int pos) {
    if (phase == 0) {
      av[m] = load_stream(acc, pos);
      cv[m] = c0 ? at32(c0, pos) : 0u;
    } else {
      cv[m] = add ? at32(add, pos) : 0u;
    }
  }
  __device__ __forceinline__ void finish(int m, int pos, uint32_t v) {
    if (phase == 0) {
      uint32_t x = mul_shoup(sub_mod(av[m], v, r), pinv, pinvp, r);
      if (c0) x = add_mod(x, cv[m], r);
      asm volatile("" : "+v"(x));  // computed here: only o stays live into the second pass
      o[m] = x;
    } else {
      uint32_t x = o[m];
      if (add) x = add_mod(x, cv[m], r);
      store_stream(dst, pos, mul_shoup(sub_mod(x, v, r), inv, invp, r));
    }
  }
};

struct MdRsArgs {
  ModDownArgs M;         // polys = 2, variant 1, c0 = d0
  const uint32_t* tmp;   // rescale column-pass output [2 batch][l'][N]
  const uint32_t* add1;  // d1 of pair b at add1 + b * add_stride
  uint64_t add_stride;
  uint32_t* out;         // [batch][2][l'][N]
  uint32_t inv[kMaxRescaleLimbs], invp[kMaxRescaleLimbs];
};

template <int LOGN, bool EARLY>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_md_rs_blk(MdRsArgs A) {
  using C = Cfg<LOGN>;
  const ModDownArgs& M = A.M;
  const int lp = M.level - 1, lk = M.level + M.K;
  const size_t ip = blockIdx.y / lp, i = blockIdx.y % lp;  // ip = 2 b + u
  const size_t b = ip >> 1, u = ip & 1;
  const size_t pi = (size_t)M.variant * M.L + i;
  MdRsLimb<(1 << C::LEB)> L;
  L.r = M.T.r[i];
  L.rinv = M.T.rinv[i];
  L.tw = M.T.tw_fblk + i * M.N;
  L.pinv = M.LT.md_pinv[pi];
  L.pinvp = M.LT.md_pinvp[pi];
  L.inv = A.inv[i];
  L.invp = A.invp[i];
  L.src_md = M.tmp2 + (ip * M.level + i) * M.N;
  L.src_rs = A.tmp + (ip * lp + i) * M.N;
  L.acc = M.acc + (ip * lk + i) * M.N;
  L.c0 = (u == 0 && M.c0 != nullptr) ? M.c0 + b * M.ct_stride + i * M.N : nullptr;
  L.add = (u == 1 && A.add1 != nullptr) ? A.add1 + b * A.add_stride + i * M.N : nullptr;
  L.dst = A.out + (ip * lp + i) * M.N;
  L.phase = 0;
  fwd_blk_pass_fetch<C::LRC, C::LRB, C::LEB, C::CB, EARLY>(L, blockIdx.x * C::CB);
  // the second pass reuses the LDS tile; the empty asm keeps its loads (and
  // the registers they take) out of the first pass
  asm volatile("" ::: "memory");
  __syncthreads();
  {
    // opaque copies: the second pass's loads cannot be hoisted into the first
    const uint32_t* src = L.src_rs;
    const uint32_t* tw = L.tw;
    asm volatile("" : "+s"(src), "+s"(tw)::"memory");
    L.src_rs = src;
    L.tw = tw;
  }
  L.phase = 1;
  fwd_blk_pass_fetch<C::LRC, C::LRB, C::LEB, C::CB, EARLY>(L, blockIdx.x * C::CB);
}

template <int LOGN, bool EARLY>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_rs_blk(RescaleArgs A) {
  using C = Cfg<LOGN>;
  const int u = blockIdx.y / A.lp, i = blockIdx.y % A.lp;
  const size_t b = u >> 1, v = u & 1;
  const uint32_t* cu = A.c + b * A.c_stride + v * A.c1_off + (size_t)i * A.N;
  const uint32_t* add = (v == 1 && A.add1 != nullptr) ? A.add1 + b * A.add_stride + (size_t)i * A.N : nullptr;
  RescaleOutLimb<(1 << C::LEB)> L{A.T.r[i],
                                  A.T.rinv[i],
                                  A.inv[i],
                                  A.invp[i],
                                  A.T.tw_fblk + (size_t)i * A.N,
                                  A.tmp + ((size_t)u * A.lp + i) * A.N,
                                  cu,
                                  add,
                                  A.out + ((size_t)u * A.lp + i) * A.N,
                                  {}};
  fwd_blk_pass_fetch<C::LRC, C::LRB, C::LEB, C::CB, EARLY>(L, blockIdx.x * C::CB);
}

// ---------------------------------------------------------------------------
// baby-step/giant-step linear transform, double hoisted
// ---------------------------------------------------------------------------
// One thread owns 4 consecutive positions of one limb t of the extended basis
// (q_0..q_{l-1}, p_0..p_{K-1}). Values enter Montgomery form (x 2^32) once, so
// each plaintext product is one REDC and pairs of products share it.
constexpr int kBsgsThreads = 256;
constexpr int kMaxBaby = 8;         // n1 (baby steps, identity included)
constexpr int kMaxGiant = 32;       // n2 (giant steps, identity included)
constexpr int kMaxBsgsLimbs = 64;   // l + K

struct BsgsArgs {
  DevTables T;
  const uint32_t* c;      // ciphertext [2][l][N]
  const uint32_t* acc;    // baby inner products [n1-1][2][l+K][N], carrying 2^-64
  const uint32_t* diag;   // [n2][n1][l+K][N] plaintext diagonals
  uint32_t* inner;        // [2][n2][l+K][N]
  const uint32_t* accg;   // giant inner products [n2-1][2][l+K][N], carrying 2^-64
  uint32_t* accqp;        // [2][l+K][N]
  int N, level, K, L, n2;
  int split;                            // 0: grid (tiles, limbs); else the 1-D walk of limb_xcd_decode
  uint32_t galois[kMaxGiant];           // baby (n1-1) or giant (n2-1) Galois elements
  uint32_t pm[kMaxBsgsLimbs];           // P 2^64 mod r_t on the q-limbs (REDC(c pm) = P c in Montgomery form)
  uint32_t m96[kMaxBsgsLimbs];          // 2^96 mod r_t (REDC(acc m96) = 2^64 acc)
  uint32_t m128[kMaxBsgsLimbs];         // 2^128 mod r_t (REDC(acc m128) = 2^64 acc in Montgomery form)
};

__device__ __forceinline__ void load4(const uint32_t* base, int pos, uint32_t (&v)[4]) {
  const uint4 x = *reinterpret_cast<const uint4*>(&at32(base, pos));
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
}

__device__ __forceinline__ void store4(uint32_t* base, int pos, const uint32_t (&v)[4]) {
  *reinterpret_cast<uint4*>(&at32(base, pos)) = make_uint4(v[0], v[1], v[2], v[3]);
}

// inner_j,u = sum_i diag[j][i] R_i,u for every giant step j, with
// R_0 = (P c0, P c1) and R_i = (P phi_{g_i}(c0) + 2^64 acc_i,0, 2^64 acc_i,1)
// (P vanishes on the p-limbs).
template <int N1>
__global__ void __launch_bounds__(kBsgsThreads) k_bsgs_baby(BsgsArgs A) {
  const int lk = A.level + A.K;
  int tile = (int)blockIdx.x, t = (int)blockIdx.y, one = 0;
  if (A.split && !limb_xcd_unit(A.N / (4 * kBsgsThreads), A.split, lk, 1, tile, t, one)) return;
  const int pos = 4 * (tile * kBsgsThreads + (int)threadIdx.x);
  const bool qlimb = t < A.level;
  const size_t pj = qlimb ? (size_t)t : (size_t)(A.L + t - A.level);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj];
  const uint32_t pm = A.pm[t], m128 = A.m128[t];
  const size_t N = (size_t)A.N;
  uint32_t R[N1][2][4];  // Montgomery form
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (qlimb) {
      uint32_t c[4];
      load4(A.c + ((size_t)u * A.level + t) * N, pos, c);
#pragma unroll
      for (int k = 0; k < 4; ++k) R[0][u][k] = redc(mul_wide(c[k], pm), r, rinv);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) R[0][u][k] = 0u;
    }
  }
#pragma unroll
  for (int i = 1; i < N1; ++i) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t a[4];
      load4(A.acc + (((size_t)(i - 1) * 2 + u) * lk + t) * N, pos, a);
#pragma unroll
      for (int k = 0; k < 4; ++k) R[i][u][k] = redc(mul_wide(a[k], m128), r, rinv);
    }
    if (qlimb) {
      const uint32_t g = A.galois[i - 1], h = (g - 1) >> 1, mask = (uint32_t)A.N - 1;
      const uint32_t* c0 = A.c + (size_t)t * N;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t x = at32(c0, ((uint32_t)(pos + k) * g + h) & mask);
        R[i][0][k] = add_mod(R[i][0][k], redc(mul_wide(x, pm), r, rinv), r);
      }
    }
  }
#pragma unroll 1
  for (int j = 0; j < A.n2; ++j) {
    uint32_t d[N1][4];
#pragma unroll
    for (int i = 0; i < N1; ++i) load4(A.diag + (((size_t)j * N1 + i) * lk + t) * N, pos, d[i]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i + 1 < N1; i += 2)
          sum = add_mod(sum, redc(mul_wide(d[i][k], R[i][u][k]) + mul_wide(d[i + 1][k], R[i + 1][u][k]), r, rinv), r);
        if constexpr (N1 % 2) sum = add_mod(sum, redc(mul_wide(d[N1 - 1][k], R[N1 - 1][u][k]), r, rinv), r);
        o[k] = sum;
      }
      store4(A.inner + (((size_t)u * A.n2 + j) * lk + t) * N, pos, o);
    }
  }
}

// acc = inner_0 + sum_{j>=1} (phi_{G_j}(inner_j,0) on the first component + 2^64 accg_j)
#if PC_IN_PART(5)
__global__ void __launch_bounds__(kBsgsThreads) k_bsgs_giant(BsgsArgs A) {
  const int lk = A.level + A.K;
  int tile = (int)blockIdx.x, t = (int)blockIdx.y, one = 0;
  if (A.split && !limb_xcd_unit(A.N / (4 * kBsgsThreads), A.split, lk, 1, tile, t, one)) return;
  const int pos = 4 * (tile * kBsgsThreads + (int)threadIdx.x);
  const size_t pj = t < A.level ? (size_t)t : (size_t)(A.L + t - A.level);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj], m96 = A.m96[t];
  const size_t N = (size_t)A.N;
  uint32_t o[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) load4(A.inner + (((size_t)u * A.n2) * lk + t) * N, pos, o[u]);
#pragma unroll 1
  for (int j = 1; j < A.n2; ++j) {
    const uint32_t g = A.galois[j - 1], h = (g - 1) >> 1, mask = (uint32_t)A.N - 1;
    const uint32_t* in0 = A.inner + ((size_t)j * lk + t) * N;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t a[4];
      load4(A.accg + (((size_t)(j - 1) * 2 + u) * lk + t) * N, pos, a);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[u][k] = add_mod(o[u][k], redc(mul_wide(a[k], m96), r, rinv), r);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) o[0][k] = add_mod(o[0][k], at32(in0, ((uint32_t)(pos + k) * g + h) & mask), r);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) store4(A.accqp + ((size_t)u * lk + t) * N, pos, o[u]);
}
#endif

// ---------------------------------------------------------------------------
// key generation: b_d[j] = -a_d[j] s[j] + e_d[j] + g_{d,j} s'[j] (mod r_j)
// One thread per 8 consecutive positions of limb j (one ChaCha block per
// digit). s'[j] is s^2 (Galois element 1) or s at the automorphism's source
// index. Products use REDC with Montgomery-form operands: S = s 2^64, so that
// REDC(a 2^-32 * S) = a s; g 2^32 mod r_j comes precomputed.
// ---------------------------------------------------------------------------
struct KeygenArgs {
  DevTables T;
  const uint32_t* s;  // [lk][N] evaluation form
  const uint32_t* e;  // [beta][lk][N] evaluation form
  uint32_t* b;        // [beta][lk][N]
  ChaChaKey seed;
  int N, level, K, L, alpha, beta;
  uint32_t galois;
  uint32_t gm[kMaxLimbsPerLaunch];  // [P]_{q_j} 2^32 mod q_j on q-limbs
};

template <int ROUNDS>
__global__ void __launch_bounds__(256) k_keygen(KeygenArgs A) {
  const int j = blockIdx.y, lk = A.level + A.K;
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= A.N) return;
  const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj], r2 = A.T.r2[pj];
  const uint32_t* sj = A.s + (size_t)j * A.N;
  const uint32_t g = A.galois, h = (g - 1) >> 1, mask = (uint32_t)A.N - 1;
  uint32_t S[8], gs[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t sv = sj[i0 + k];
    const uint32_t s1 = redc(mul_wide(sv, r2), r, rinv);                   // s 2^32
    S[k] = redc(mul_wide(s1, r2), r, rinv);                                // s 2^64
    const uint32_t sp = g == 1u ? redc(mul_wide(sv, s1), r, rinv)          // s^2
                                : sj[((uint32_t)(i0 + k) * g + h) & mask];  // phi_g(s)
    gs[k] = redc(mul_wide(sp, A.gm[j]), r, rinv);                          // g s'
  }
  for (int d = 0; d < A.beta; ++d) {
    const bool own = j < A.level && j >= d * A.alpha && j < (d + 1) * A.alpha;
    uint32_t w[16];
    chacha_block<ROUNDS>(A.seed, (uint32_t)(i0 >> 3), 0u, (uint32_t)d, (uint32_t)j, w);
    const uint32_t* ed = A.e + ((size_t)d * lk + j) * A.N + i0;
    uint32_t* bd = A.b + ((size_t)d * lk + j) * A.N + i0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t am = word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv);  // a 2^-32
      uint32_t t = sub_mod(ed[k], redc(mul_wide(am, S[k]), r, rinv), r);        // e - a s
      if (own) t = add_mod(t, gs[k], r);
      bd[k] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define PC_DISPATCH_LOGN(logn, ...) \
  switch (logn) {                   \
    case 12: {                      \
      constexpr int LN = 12;        \
      __VA_ARGS__;                  \
      break;                        \
    }                               \
    case 16: {                      \
      constexpr int LN = 16;        \
      __VA_ARGS__;                  \
      break;                        \
    }                               \
    case 17: {                      \
      constexpr int LN = 17;        \
      __VA_ARGS__;                  \
      break;                        \
    }                               \
    default:                        \
      return hipErrorInvalidValue;  \
  }

// CNT = x for x in 1..kMaxAlpha (= kMaxSpecial)
#define PC_DISPATCH_CNT(x, ...)                         \
  switch (x) {                                          \
    case 1: { constexpr int CNT = 1; __VA_ARGS__; break; } \
    case 2: { constexpr int CNT = 2; __VA_ARGS__; break; } \
    case 3: { constexpr int CNT = 3; __VA_ARGS__; break; } \
    case 4: { constexpr int CNT = 4; __VA_ARGS__; break; } \
    case 5: { constexpr int CNT = 5; __VA_ARGS__; break; } \
    case 6: { constexpr int CNT = 6; __VA_ARGS__; break; } \
    case 7: { constexpr int CNT = 7; __VA_ARGS__; break; } \
    case 8: { constexpr int CNT = 8; __VA_ARGS__; break; } \
    default: return hipErrorInvalidValue;               \
  }
static_assert(kMaxAlpha == 8 && kMaxSpecial == 8, "PC_DISPATCH_CNT covers 1..8");

#if PC_IN_PART(1)
hipError_t launch_ntt(const pc_params* p, uint32_t* data, uint32_t* tmp, const uint32_t* prime_idx, uint32_t nlimbs,
                      bool inverse, hipStream_t s) {
  for (uint32_t base = 0; base < nlimbs; base += kMaxLimbsPerLaunch) {
    const uint32_t cnt = (nlimbs - base) < (uint32_t)kMaxLimbsPerLaunch ? (nlimbs - base) : kMaxLimbsPerLaunch;
    NttArgs A;
    A.T = p->tabs;
    A.data = data + (size_t)base * p->N;
    A.tmp = tmp + (size_t)base * p->N;
    A.N = (int)p->N;
    for (uint32_t z = 0; z < cnt; ++z) A.pidx[z] = (uint8_t)prime_idx[base + z];
    PC_DISPATCH_LOGN(p->log2n, {
      if (!inverse) {
        { LaunchTimer tm(p, KID_NTT_FWD_COL, s); hipLaunchKernelGGL(k_ntt_fwd_col<LN>, dim3(col_tiles<LN>(), cnt), dim3(col_threads<LN>()), 0, s, A); }
        { LaunchTimer tm(p, KID_NTT_FWD_BLK, s); hipLaunchKernelGGL(k_ntt_fwd_blk<LN>, dim3(blk_tiles<LN>(), cnt), dim3(blk_threads<LN>()), 0, s, A); }
      } else {
        { LaunchTimer tm(p, KID_NTT_INV_BLK, s); hipLaunchKernelGGL(k_ntt_inv_blk<LN>, dim3(blk_tiles<LN>(), cnt), dim3(blk_threads<LN>()), 0, s, A); }
        { LaunchTimer tm(p, KID_NTT_INV_COL, s); hipLaunchKernelGGL(k_ntt_inv_col<LN>, dim3(col_tiles<LN>(), cnt), dim3(col_threads<LN>()), 0, s, A); }
      }
    });
  }
  return hipGetLastError();
}

hipError_t launch_modup(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset, uint32_t batch,
                        uint32_t level, const KsWorkspace& ws, hipStream_t s, bool fwd_blk) {
  ModUpArgs A;
  A.T = p->tabs;
  A.LT = p->ltabs;
  A.ct = ct;
  A.ct_stride = ct_stride;
  A.c1_off = c1_offset;
  A.y = ws.y;
  A.ys = (int)(p->N + kLimbPad);
  A.tmp = ws.tmp;
  A.ext = ws.ext;
  A.N = (int)p->N;
  A.level = (int)level;
  A.K = (int)p->K;
  A.L = (int)p->L;
  A.alpha = alpha_of(p, level);
  A.beta = beta_of(p, level);
  A.scale_off = p->mu_scale_off[level];
  A.bconv_off = p->mu_bconv_off[level];
  A.batch = (int)batch;
  A.seg = ws.seg ? 1 : 0;
  const uint32_t rows_in = batch * level;
  const uint32_t rows_ext = batch * (uint32_t)A.beta * (level + p->K);
  // the last digit is the shortest, so it has the most targets
  const int targets = (int)(level + p->K) - ((int)level - (A.beta - 1) * A.alpha);
  const int tiles_c = col_tiles_of(p->log2n);
  const bool one = xcd_grid(tiles_c, (int)batch * A.beta, (targets + kBconvGroup - 1) / kBconvGroup) < kBconvSmallGrid;
  const int G = one ? 1 : kBconvGroup;
  const uint32_t groups = (uint32_t)((targets + G - 1) / G);
  A.ngroups = (int)groups;
  PC_DISPATCH_LOGN(p->log2n, {
    { LaunchTimer tm(p, KID_MODUP_INV_BLK, s); hipLaunchKernelGGL(k_modup_inv_blk<LN>, dim3(blk_tiles<LN>(), rows_in), dim3(blk_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODUP_INV_COL, s); hipLaunchKernelGGL(k_modup_inv_col<LN>, dim3(col_tiles<LN>(), rows_in), dim3(col_threads<LN>()), 0, s, A); }
    PC_DISPATCH_CNT(A.alpha, {
      LaunchTimer tm(p, KID_MODUP_BCONV, s);
      const dim3 grid(xcd_grid(col_tiles<LN>(), (int)batch * A.beta, (int)groups));
      if (one)
        hipLaunchKernelGGL((k_modup_bconv<LN, CNT, 1>), grid, dim3(col_threads<LN>()), 0, s, A);
      else
        hipLaunchKernelGGL((k_modup_bconv<LN, CNT, kBconvGroup>), grid, dim3(col_threads<LN>()), 0, s, A);
    });
    if (fwd_blk) { LaunchTimer tm(p, KID_MODUP_FWD_BLK, s); hipLaunchKernelGGL(k_modup_fwd_blk<LN>, dim3(blk_tiles<LN>(), rows_ext), dim3(blk_threads<LN>()), 0, s, A); }
  });
  return hipGetLastError();
}

#endif
// Workgroups of `kernel` resident on the current device at once, cached per
// (kernel, device) in a fixed table (no allocation after the first lookup).
template <class F>
static uint32_t resident_workgroups(F kernel, int threads) {
  struct Entry {
    const void* kernel;
    int dev;
    uint32_t n;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const void* kp = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].kernel == kp && cache[i].dev == dev) return cache[i].n;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
  const uint32_t n = (uint32_t)(per_cu * cus);
  if (used < 64) cache[used++] = Entry{kp, dev, n};
  return n;
}

// Split of limb_xcd_decode for `limbs` limbs of `tiles` tiles: the smallest of
// 1, 2, 4, 8 (dividing tiles) whose padding to a multiple of 8 parts costs at
// most 7%, else the one with the least padding.
[[maybe_unused]] static int xcd_split(uint32_t limbs, uint32_t tiles) {
  int best = 1;
  double best_pad = 1e9;
  for (uint32_t sp = 1; sp <= 8 && sp <= tiles; sp *= 2) {
    if (tiles % sp) break;
    const uint32_t parts = limbs * sp, padded = (parts + 7) / 8 * 8;
    const double pad = (double)padded / parts;
    if (pad <= 1.07) return (int)sp;
    if (pad < best_pad) {
      best_pad = pad;
      best = (int)sp;
    }
  }
  return best;
}

[[maybe_unused]] static uint32_t blk_tiles_of(uint32_t log2n) {
  return log2n == 12 ? (uint32_t)blk_tiles<12>() : log2n == 16 ? (uint32_t)blk_tiles<16>() : (uint32_t)blk_tiles<17>();
}

#if PC_IN_PART(2)
template <int BETA, int ROUNDS, int BT>
static void launch_ip_regen(const pc_params* p, const IPArgs& A0, bool seg, hipStream_t s) {
  auto kern = seg ? k_ip_regen<BETA, ROUNDS, BT, true> : k_ip_regen<BETA, ROUNDS, BT, false>;
  const uint32_t lk = (uint32_t)(A0.level + A0.K), tiles = p->N / (8 * kIpHalf);
  IPArgs A = A0;
  if (A.limb_xcd) A.limb_xcd = xcd_split(lk, tiles);
  const uint32_t sp = (uint32_t)A.limb_xcd;
  const uint32_t units = sp ? 8 * ((lk * sp + 7) / 8) * (uint32_t)A.nkeys * (tiles / sp) : (uint32_t)A.nkeys * lk * tiles;
  uint32_t grid = std::min(units, resident_workgroups(kern, 2 * kIpHalf));
  if (sp) grid = std::max<uint32_t>(8, grid & ~7u);  // unit u stays on XCD u mod 8
  LaunchTimer tm(p, KID_INNER_PRODUCT, s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(2 * kIpHalf), 0, s, A);
}

template <int BETA, int BT, bool SEG>
static void launch_ip_kernel(const IPArgs& A, dim3 grid, bool stored, int rounds, hipStream_t s) {
  if (stored)
    hipLaunchKernelGGL((k_inner_product<BETA, 12, true, BT, SEG>), grid, dim3(kIpThreads), 0, s, A);
  else if (rounds == 20)
    hipLaunchKernelGGL((k_inner_product<BETA, 20, false, BT, SEG>), grid, dim3(kIpThreads), 0, s, A);
  else
    hipLaunchKernelGGL((k_inner_product<BETA, 12, false, BT, SEG>), grid, dim3(kIpThreads), 0, s, A);
}

// Source bytes per limb above which a gathering batch takes one workgroup per
// inner-product unit (4 x an XCD's 4 MB L2).
constexpr size_t kGatherSetBytes = size_t(16) << 20;

template <int BETA, int BT>
static void launch_ip_bt(const pc_params* p, const IPArgs& A0, uint32_t nkeys, bool stored, bool seg,
                         hipStream_t s) {
  if constexpr (BT != 1) {
    // regenerated a half and a batch to overlap it with: the producer/consumer
    // kernel, unless the call gathers from more than kGatherSetBytes of
    // sources per limb (batch x digits x limb bytes), where its persistent walk
    // refetches them more than one workgroup per unit does (measured: the
    // N = 2^17 relinearise-and-rotate chain, 20 MB, 3.57K -> 3.68K key
    // switches/s; the N = 2^16 level sweep, 8 MB, slower)
    const size_t gather_set = (size_t)A0.batch * BETA * p->N * 4;
    if (!stored && A0.batch >= 2 && (A0.limb_xcd == 0 || gather_set <= kGatherSetBytes)) {
      if (p->chacha_rounds == 20)
        launch_ip_regen<BETA, 20, BT>(p, A0, seg, s);
      else
        launch_ip_regen<BETA, 12, BT>(p, A0, seg, s);
      return;
    }
  }
  const uint32_t tiles = (p->N / 8 + kIpThreads - 1) / kIpThreads, lk = (uint32_t)(A0.level + A0.K);
  IPArgs A = A0;
  if (A.limb_xcd) A.limb_xcd = xcd_split(lk, tiles);
  const uint32_t sp = (uint32_t)A.limb_xcd;
  const dim3 grid = sp ? dim3(8 * ((lk * sp + 7) / 8) * nkeys * (tiles / sp)) : dim3(tiles, lk, nkeys);
  LaunchTimer tm(p, KID_INNER_PRODUCT, s);
  if (seg)
    launch_ip_kernel<BETA, BT, true>(A, grid, stored, (int)p->chacha_rounds, s);
  else
    launch_ip_kernel<BETA, BT, false>(A, grid, stored, (int)p->chacha_rounds, s);
}

template <int BETA>
static void launch_ip_beta(const pc_params* p, const IPArgs& A, uint32_t nkeys, bool stored, bool seg,
                           hipStream_t s) {
  if (A.batch == 8)
    launch_ip_bt<BETA, 8>(p, A, nkeys, stored, seg, s);
  else if (A.batch == 1)
    launch_ip_bt<BETA, 1>(p, A, nkeys, stored, seg, s);
  else
    launch_ip_bt<BETA, 0>(p, A, nkeys, stored, seg, s);
}

hipError_t launch_inner_product(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset,
                                uint32_t batch, uint32_t level, const KsWorkspace& ws, const KeyRef* keys,
                                uint32_t nkeys, hipStream_t s, bool one_ct_per_key) {
  const int beta = beta_of(p, level);
  for (uint32_t base = 0; base < nkeys; base += kMaxKeysPerLaunch) {
    const uint32_t cnt = (nkeys - base) < (uint32_t)kMaxKeysPerLaunch ? (nkeys - base) : kMaxKeysPerLaunch;
    IPArgs A;
    A.T = p->tabs;
    A.ct = ct;
    A.ct_stride = ct_stride;
    A.c1_off = c1_offset;
    A.ext = ws.ext;
    A.acc = ws.acc;
    A.N = (int)p->N;
    A.level = (int)level;
    A.K = (int)p->K;
    A.L = (int)p->L;
    A.alpha = alpha_of(p, level);
    A.batch = (int)batch;
    A.nkeys = (int)cnt;
    A.key_level = (int)key_level_of(p, level);
    A.key_base = base;
    A.ct_key_stride = one_ct_per_key ? ct_stride * batch : 0;
    A.ext_key_stride = one_ct_per_key ? (uint64_t)batch * beta * (level + p->K) * p->N : 0;
    A.lrc = pass_split_lrc(p->log2n);
    A.lrb = (int)p->log2n - A.lrc;
    bool stored = false;
    A.limb_xcd = 0;
    for (uint32_t k = 0; k < cnt; ++k) {
      const KeyRef& kr = keys[base + k];
      if (kr.galois != 1u) A.limb_xcd = -1;  // split chosen below, per kernel
      A.evk_b[k] = kr.b;
      A.evk_a[k] = kr.a;
      stored = stored || kr.a != nullptr;
      for (int w = 0; w < 8; ++w) A.seed[k].k[w] = kr.seed[w];
      A.galois[k] = kr.galois;
    }
    switch (beta) {
      case 1: launch_ip_beta<1>(p, A, cnt, stored, ws.seg, s); break;
      case 2: launch_ip_beta<2>(p, A, cnt, stored, ws.seg, s); break;
      case 3: launch_ip_beta<3>(p, A, cnt, stored, ws.seg, s); break;
      case 4: launch_ip_beta<4>(p, A, cnt, stored, ws.seg, s); break;
      case 5: launch_ip_beta<5>(p, A, cnt, stored, ws.seg, s); break;
      case 6: launch_ip_beta<6>(p, A, cnt, stored, ws.seg, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

#endif
#if PC_IN_PART(3)
template <int LN, int BETA>
static void launch_modup_ip_kernel(const pc_params* p, const ModUpIPArgs& A, dim3 grid, hipStream_t s) {
  if constexpr (BETA * (1 << Cfg<LN>::LEB) <= kFusedKeyValues) {
    const dim3 block(fused_threads<LN>());
    if (A.evk_a != nullptr)
      hipLaunchKernelGGL((k_modup_ip<LN, BETA, 12, true>), grid, block, 0, s, A);
    else if (p->chacha_rounds == 20)
      hipLaunchKernelGGL((k_modup_ip<LN, BETA, 20, false>), grid, block, 0, s, A);
    else
      hipLaunchKernelGGL((k_modup_ip<LN, BETA, 12, false>), grid, block, 0, s, A);
  }
}

hipError_t launch_modup_ip(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset,
                           uint32_t batch, uint32_t level, const KsWorkspace& ws, const KeyRef* keys, uint32_t nkeys,
                           hipStream_t s) {
  const int beta = beta_of(p, level);
  const int per_thread = p->log2n == 16 ? 1 << Cfg<16>::LEB : p->log2n == 17 ? 1 << Cfg<17>::LEB : 1 << Cfg<12>::LEB;
  const bool fused = nkeys == 1 && keys[0].galois == 1u && !ws.seg && beta * per_thread <= kFusedKeyValues;
  hipError_t e = launch_modup(p, ct, ct_stride, c1_offset, batch, level, ws, s, !fused);
  if (e != hipSuccess || !fused) return e != hipSuccess ? e : launch_inner_product(p, ct, ct_stride, c1_offset, batch,
                                                                                   level, ws, keys, nkeys, s);
  ModUpIPArgs A;
  A.T = p->tabs;
  A.ct = ct;
  A.ct_stride = ct_stride;
  A.c1_off = c1_offset;
  A.tmp = ws.tmp;
  A.acc = ws.acc;
  A.evk_b = keys[0].b;
  A.evk_a = keys[0].a;
  for (int w = 0; w < 8; ++w) A.seed.k[w] = keys[0].seed[w];
  A.N = (int)p->N;
  A.level = (int)level;
  A.K = (int)p->K;
  A.L = (int)p->L;
  A.alpha = alpha_of(p, level);
  A.batch = (int)batch;
  A.key_level = (int)key_level_of(p, level);
  const int lk = (int)(level + p->K);
  LaunchTimer tm(p, KID_MODUP_IP, s);
  PC_DISPATCH_LOGN(p->log2n, {
    constexpr int CF = fused_cols<LN>(), G = 32 / CF;
    const dim3 grid(xcd_grid((1 << Cfg<LN>::LRC) / CF / G, lk, G));
    switch (beta) {
      case 1: launch_modup_ip_kernel<LN, 1>(p, A, grid, s); break;
      case 2: launch_modup_ip_kernel<LN, 2>(p, A, grid, s); break;
      case 3: launch_modup_ip_kernel<LN, 3>(p, A, grid, s); break;
      case 4: launch_modup_ip_kernel<LN, 4>(p, A, grid, s); break;
      case 5: launch_modup_ip_kernel<LN, 5>(p, A, grid, s); break;
      case 6: launch_modup_ip_kernel<LN, 6>(p, A, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  });
  return hipGetLastError();
}

#endif
// Fetch the side inputs of a combining block pass after the transform when the
// grid has at least 8 polynomials of rows (measured: ModDown combine of 8 key
// switches 87 -> 84 us, rescale of 8 products 96 -> 83 us); smaller grids and
// gathers keep the early fetch, which hides their latency better.
[[maybe_unused]] static bool late_fetch(uint32_t polys) { return polys >= 8; }

#if PC_IN_PART(4)
hipError_t launch_seg_copy(const pc_params* p, const uint32_t* src, uint32_t limbs, uint32_t* dst, hipStream_t s) {
  SegCopyArgs A;
  A.src = src;
  A.dst = dst;
  A.N = (int)p->N;
  PC_DISPATCH_LOGN(p->log2n, {
    LaunchTimer tm(p, KID_SEG_COPY, s);
    hipLaunchKernelGGL(k_seg_copy<LN>, dim3(blk_tiles<LN>(), limbs), dim3(blk_threads<LN>()), 0, s, A);
  });
  return hipGetLastError();
}

hipError_t launch_moddown(const pc_params* p, const uint32_t* acc, uint32_t items, uint32_t polys, uint32_t level,
                          int variant, uint32_t* out, const KsWorkspace& ws, const uint32_t* c0, uint64_t ct_stride,
                          uint32_t batch, const uint32_t* galois_per_key, hipStream_t s, bool c0_seg,
                          uint32_t combine_from) {
  if (combine_from >= level) return hipErrorInvalidValue;
  ModDownArgs A;
  A.T = p->tabs;
  A.LT = p->ltabs;
  A.acc = acc;
  A.y2 = ws.y2;
  A.y2s = (int)(p->N + kLimbPad);
  A.tmp2 = ws.tmp2;
  A.out = out;
  A.c0 = c0;
  A.ct_stride = ct_stride;
  A.N = (int)p->N;
  A.level = (int)level;
  A.K = (int)p->K;
  A.L = (int)p->L;
  A.polys = (int)polys;
  A.variant = variant;
  A.batch = (int)(batch ? batch : 1);
  const uint32_t nkeys = items / A.batch;
  if (c0 != nullptr && nkeys > (uint32_t)kMaxKeysPerLaunch) return hipErrorInvalidValue;
  for (uint32_t k = 0; k < (uint32_t)kMaxKeysPerLaunch; ++k)
    A.galois[k] = (galois_per_key != nullptr && k < nkeys) ? galois_per_key[k] : 1u;
  const uint32_t rows_p = items * polys * p->K;
  A.i0 = (int)combine_from;
  A.ni = (int)(level - combine_from);
  const uint32_t rows_q = items * polys * (uint32_t)A.ni;
  const int tiles_c = col_tiles_of(p->log2n);
  const bool one = xcd_grid(tiles_c, (int)(items * polys), (int)((level + kBconvGroup - 1) / kBconvGroup)) <
                   kBconvSmallGrid;
  const uint32_t G = one ? 1u : (uint32_t)kBconvGroup;
  const uint32_t groups = (level + G - 1) / G;
  A.rows_ip = (int)(items * polys);
  A.ngroups = (int)groups;
  A.limb_xcd = 0;
  if (c0 != nullptr)
    for (uint32_t k = 0; k < nkeys && k < (uint32_t)kMaxKeysPerLaunch; ++k)
      if (A.galois[k] != 1u) A.limb_xcd = xcd_split(level, (uint32_t)blk_tiles_of(p->log2n));
  if (A.limb_xcd && combine_from != 0) return hipErrorInvalidValue;  // the XCD walk covers whole polynomials
  PC_DISPATCH_LOGN(p->log2n, {
    { LaunchTimer tm(p, KID_MODDOWN_INV_BLK, s); hipLaunchKernelGGL(k_md_inv_blk<LN>, dim3(blk_tiles<LN>(), rows_p), dim3(blk_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODDOWN_INV_COL, s); hipLaunchKernelGGL(k_md_inv_col<LN>, dim3(col_tiles<LN>(), rows_p), dim3(col_threads<LN>()), 0, s, A); }
    PC_DISPATCH_CNT(A.K, {
      LaunchTimer tm(p, KID_MODDOWN_BCONV, s);
      const dim3 grid(xcd_grid(col_tiles<LN>(), (int)(items * polys), (int)groups));
      if (one)
        hipLaunchKernelGGL((k_md_bconv<LN, CNT, 1>), grid, dim3(col_threads<LN>()), 0, s, A);
      else
        hipLaunchKernelGGL((k_md_bconv<LN, CNT, kBconvGroup>), grid, dim3(col_threads<LN>()), 0, s, A);
    });
    {
      const uint32_t sp = (uint32_t)A.limb_xcd;
      const dim3 grid = sp ? dim3(8 * ((level * sp + 7) / 8) * items * polys * (blk_tiles<LN>() / sp))
                           : dim3(blk_tiles<LN>(), rows_q);
      LaunchTimer tm(p, KID_MODDOWN_FWD_BLK, s);
      const dim3 bt(blk_threads<LN>());
      bool gather = false;
      for (uint32_t k = 0; k < nkeys && k < (uint32_t)kMaxKeysPerLaunch; ++k) gather = gather || A.galois[k] != 1u;
      if (c0 == nullptr) {
        if (late_fetch(items * polys))
          hipLaunchKernelGGL((k_md_fwd_blk<LN, kNoC0, false>), grid, bt, 0, s, A);
        else
          hipLaunchKernelGGL((k_md_fwd_blk<LN, kNoC0, true>), grid, bt, 0, s, A);
      } else if (c0_seg) {
        hipLaunchKernelGGL((k_md_fwd_blk<LN, kC0Seg, true>), grid, bt, 0, s, A);
      } else if (gather) {
        hipLaunchKernelGGL((k_md_fwd_blk<LN, kC0Gather, true>), grid, bt, 0, s, A);
      } else if (late_fetch(items * polys)) {
        hipLaunchKernelGGL((k_md_fwd_blk<LN, kC0Same, false>), grid, bt, 0, s, A);
      } else {
        hipLaunchKernelGGL((k_md_fwd_blk<LN, kC0Same, true>), grid, bt, 0, s, A);
      }
    }
  });
  return hipGetLastError();
}

#endif
#if PC_IN_PART(5)
hipError_t launch_tensor(const pc_params* p, const uint32_t* a, uint64_t a_stride, const uint32_t* b,
                         uint64_t b_stride, uint32_t batch, uint32_t level, uint32_t* d, uint64_t d_stride,
                         const uint64_t d_off[3], hipStream_t s) {
  TensorArgs A;
  A.T = p->tabs;
  A.a = a;
  A.b = b;
  A.a_stride = a_stride;
  A.b_stride = b_stride;
  A.d = d;
  A.d_stride = d_stride;
  for (int k = 0; k < 3; ++k) A.d_off[k] = d_off[k];
  A.N = (int)p->N;
  A.level = (int)level;
  const dim3 grid(p->N / (8 * kTensorThreads), level, batch);
  LaunchTimer tm(p, KID_TENSOR, s);
  hipLaunchKernelGGL(k_tensor, grid, dim3(kTensorThreads), 0, s, A);
  return hipGetLastError();
}

// q_{l'}^-1 mod q_i and its Shoup companion for i < l' = level - 1.
static void rescale_inverses(const pc_params* p, uint32_t level, uint32_t* inv, uint32_t* invp) {
  const uint32_t lp = level - 1;
  const size_t off = (size_t)lp * p->L;  // rows of the per-level rescale tables
  for (uint32_t i = 0; i < (uint32_t)kMaxRescaleLimbs; ++i) {
    inv[i] = i < lp ? p->h_rs_inv[off + i] : 0u;
    invp[i] = i < lp ? p->h_rs_invp[off + i] : 0u;
  }
}

hipError_t launch_rescale(const pc_params* p, const uint32_t* c, uint64_t c_stride, uint32_t c1_off,
                          const uint32_t* add1, uint64_t add_stride, uint32_t batch, uint32_t level, uint32_t* x,
                          uint32_t* tmp, uint32_t* out, hipStream_t s, bool final_pass) {
  const uint32_t lp = level - 1, polys = 2 * batch;
  if (level < 2 || lp > (uint32_t)kMaxRescaleLimbs || polys > (uint32_t)kMaxLimbsPerLaunch) return hipErrorInvalidValue;
  RescaleArgs A;
  A.T = p->tabs;
  A.x = x;
  A.c = c;
  A.c_stride = c_stride;
  A.c1_off = c1_off;
  A.add1 = add1;
  A.add_stride = add_stride;
  A.x_out = x;
  A.tmp = tmp;
  A.out = out;
  A.N = (int)p->N;
  A.lp = (int)lp;
  A.ql_half = p->primes[lp] / 2;
  const size_t off = (size_t)lp * p->L;  // rows of the per-level rescale tables
  for (uint32_t i = 0; i < (uint32_t)kMaxRescaleLimbs; ++i) A.ql_mod[i] = i < lp ? p->h_rs_qlmod[off + i] : 0u;
  rescale_inverses(p, level, A.inv, A.invp);
  {
    LaunchTimer tm(p, KID_RESCALE_GATHER, s);
    hipLaunchKernelGGL(k_rs_gather, dim3(p->N / (4 * kGatherThreads), polys), dim3(kGatherThreads), 0, s, A);
  }
  // limb l' of every polynomial to coefficient form
  std::vector<uint32_t> pidx(polys, lp);
  hipError_t e = launch_ntt(p, x, tmp, pidx.data(), polys, true, s);
  if (e != hipSuccess) return e;
  const uint32_t rows = polys * lp;
  PC_DISPATCH_LOGN(p->log2n, {
    { LaunchTimer tm(p, KID_RESCALE_COL, s); hipLaunchKernelGGL(k_rs_col<LN>, dim3(col_tiles<LN>(), rows), dim3(col_threads<LN>()), 0, s, A); }
    if (final_pass) {
      LaunchTimer tm(p, KID_RESCALE_BLK, s);
      if (late_fetch(polys))
        hipLaunchKernelGGL((k_rs_blk<LN, false>), dim3(blk_tiles<LN>(), rows), dim3(blk_threads<LN>()), 0, s, A);
      else
        hipLaunchKernelGGL((k_rs_blk<LN, true>), dim3(blk_tiles<LN>(), rows), dim3(blk_threads<LN>()), 0, s, A);
    }
  });
  return hipGetLastError();
}

hipError_t launch_moddown_rescale(const pc_params* p, const uint32_t* acc, uint32_t batch, uint32_t level,
                                  const KsWorkspace& ws, const uint32_t* c0, uint64_t ct_stride,
                                  const uint32_t* add1, uint64_t add_stride, const uint32_t* tmp, uint32_t* out,
                                  hipStream_t s) {
  const uint32_t lp = level - 1, polys = 2 * batch;
  if (level < 2 || lp > (uint32_t)kMaxRescaleLimbs || polys > (uint32_t)kMaxLimbsPerLaunch) return hipErrorInvalidValue;
  MdRsArgs A;
  ModDownArgs& M = A.M;
  M.T = p->tabs;
  M.LT = p->ltabs;
  M.acc = acc;
  M.y2 = ws.y2;
  M.y2s = (int)(p->N + kLimbPad);
  M.tmp2 = ws.tmp2;
  M.out = nullptr;
  M.c0 = c0;
  M.ct_stride = ct_stride;
  M.N = (int)p->N;
  M.level = (int)level;
  M.K = (int)p->K;
  M.L = (int)p->L;
  M.polys = 2;
  M.variant = 1;  // acc carries 2^-64
  M.batch = (int)batch;
  M.rows_ip = (int)polys;
  M.ngroups = 0;
  M.limb_xcd = 0;
  M.i0 = 0;
  M.ni = (int)lp;
  for (int k = 0; k < kMaxKeysPerLaunch; ++k) M.galois[k] = 1u;
  A.tmp = tmp;
  A.add1 = add1;
  A.add_stride = add_stride;
  A.out = out;
  rescale_inverses(p, level, A.inv, A.invp);
  const uint32_t rows = polys * lp;
  PC_DISPATCH_LOGN(p->log2n, {
    LaunchTimer tm(p, KID_MODDOWN_RESCALE, s);
    if (late_fetch(polys))
      hipLaunchKernelGGL((k_md_rs_blk<LN, false>), dim3(blk_tiles<LN>(), rows), dim3(blk_threads<LN>()), 0, s, A);
    else
      hipLaunchKernelGGL((k_md_rs_blk<LN, true>), dim3(blk_tiles<LN>(), rows), dim3(blk_threads<LN>()), 0, s, A);
  });
  return hipGetLastError();
}

static void bsgs_args(const pc_params* p, BsgsArgs& A, uint32_t level, uint32_t n2, const uint32_t* galois,
                      uint32_t ngalois, const uint32_t* pm, const uint32_t* m96, const uint32_t* m128) {
  A.T = p->tabs;
  A.N = (int)p->N;
  A.level = (int)level;
  A.K = (int)p->K;
  A.L = (int)p->L;
  A.n2 = (int)n2;
  A.split = 0;
  for (uint32_t k = 0; k < (uint32_t)kMaxGiant; ++k) A.galois[k] = k < ngalois ? galois[k] : 1u;
  for (uint32_t k = 0; k < ngalois; ++k)
    if (galois[k] != 1u) A.split = xcd_split(level + p->K, p->N / (4 * kBsgsThreads));
  const uint32_t lk = level + p->K;
  for (uint32_t t = 0; t < (uint32_t)kMaxBsgsLimbs; ++t) {
    A.pm[t] = t < lk ? pm[t] : 0u;
    A.m96[t] = t < lk ? m96[t] : 0u;
    A.m128[t] = t < lk ? m128[t] : 0u;
  }
}

hipError_t launch_bsgs_baby(const pc_params* p, const uint32_t* ct, const uint32_t* acc, const uint32_t* diag,
                            uint32_t* inner, uint32_t level, uint32_t n1, uint32_t n2, const uint32_t* baby_galois,
                            const uint32_t* pm, const uint32_t* m96, const uint32_t* m128, hipStream_t s) {
  const uint32_t lk = level + p->K;
  if (n1 < 1 || n1 > (uint32_t)kMaxBaby || n2 < 1 || n2 > (uint32_t)kMaxGiant || lk > (uint32_t)kMaxBsgsLimbs)
    return hipErrorInvalidValue;
  BsgsArgs A;
  bsgs_args(p, A, level, n2, baby_galois, n1 - 1, pm, m96, m128);
  A.c = ct;
  A.acc = acc;
  A.diag = diag;
  A.inner = inner;
  A.accg = nullptr;
  A.accqp = nullptr;
  const uint32_t tiles = p->N / (4 * kBsgsThreads), sp = (uint32_t)A.split;
  const dim3 grid = sp ? dim3(8 * ((lk * sp + 7) / 8) * (tiles / sp)) : dim3(tiles, lk);
  LaunchTimer tm(p, KID_BSGS_BABY, s);
  switch (n1) {
#define PC_BSGS_CASE(n) \
  case n: hipLaunchKernelGGL(k_bsgs_baby<n>, grid, dim3(kBsgsThreads), 0, s, A); break;
    PC_BSGS_CASE(1) PC_BSGS_CASE(2) PC_BSGS_CASE(3) PC_BSGS_CASE(4)
    PC_BSGS_CASE(5) PC_BSGS_CASE(6) PC_BSGS_CASE(7) PC_BSGS_CASE(8)
#undef PC_BSGS_CASE
    default: return hipErrorInvalidValue;
  }
  static_assert(kMaxBaby == 8, "the dispatch above covers n1 = 1..8");
  return hipGetLastError();
}

hipError_t launch_bsgs_giant(const pc_params* p, const uint32_t* inner, const uint32_t* accg, uint32_t* accqp,
                             uint32_t level, uint32_t n2, const uint32_t* giant_galois, const uint32_t* pm,
                             const uint32_t* m96, const uint32_t* m128, hipStream_t s) {
  const uint32_t lk = level + p->K;
  if (n2 < 1 || n2 > (uint32_t)kMaxGiant || lk > (uint32_t)kMaxBsgsLimbs) return hipErrorInvalidValue;
  BsgsArgs A;
  bsgs_args(p, A, level, n2, giant_galois, n2 - 1, pm, m96, m128);
  A.c = nullptr;
  A.acc = nullptr;
  A.diag = nullptr;
  A.inner = const_cast<uint32_t*>(inner);
  A.accg = accg;
  A.accqp = accqp;
  const uint32_t tiles = p->N / (4 * kBsgsThreads), sp = (uint32_t)A.split;
  const dim3 grid = sp ? dim3(8 * ((lk * sp + 7) / 8) * (tiles / sp)) : dim3(tiles, lk);
  LaunchTimer tm(p, KID_BSGS_GIANT, s);
  hipLaunchKernelGGL(k_bsgs_giant, grid, dim3(kBsgsThreads), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_keygen(const pc_params* p, const uint32_t seed[8], uint32_t level, uint32_t galois,
                         const uint32_t* s_eval, const uint32_t* e_eval, const uint32_t* gm, uint32_t* evk_b,
                         hipStream_t s) {
  KeygenArgs A;
  A.T = p->tabs;
  A.s = s_eval;
  A.e = e_eval;
  A.b = evk_b;
  for (int w = 0; w < 8; ++w) A.seed.k[w] = seed[w];
  A.N = (int)p->N;
  A.level = (int)level;
  A.K = (int)p->K;
  A.L = (int)p->L;
  A.alpha = alpha_of(p, level);
  A.beta = beta_of(p, level);
  A.galois = galois;
  const uint32_t lk = level + p->K;
  for (uint32_t j = 0; j < (uint32_t)kMaxLimbsPerLaunch; ++j) A.gm[j] = j < lk ? gm[j] : 0u;
  const dim3 grid((p->N / 8 + 255) / 256, lk);
  LaunchTimer tm(p, KID_KEYGEN, s);
  if (p->chacha_rounds == 20)
    hipLaunchKernelGGL(k_keygen<20>, grid, dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL(k_keygen<12>, grid, dim3(256), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_chacha_expand(const pc_params* p, const uint32_t seed[8], uint32_t d, uint32_t j,
                                uint32_t prime_index, uint32_t* dst, hipStream_t s) {
  ChaChaKey key;
  for (int w = 0; w < 8; ++w) key.k[w] = seed[w];
  const uint32_t r = p->primes[prime_index];
  const uint32_t rinv = p->h_rinv[prime_index];
  const uint32_t r2 = p->h_r2[prime_index];
  const dim3 grid((p->N / 8 + 255) / 256);
  LaunchTimer tm(p, KID_CHACHA_EXPAND, s);
  if (p->chacha_rounds == 20)
    hipLaunchKernelGGL(k_chacha_expand<20>, grid, dim3(256), 0, s, key, d, j, r, rinv, r2, dst, (int)p->N);
  else
    hipLaunchKernelGGL(k_chacha_expand<12>, grid, dim3(256), 0, s, key, d, j, r, rinv, r2, dst, (int)p->N);
  return hipGetLastError();
}

hipError_t launch_expand_key(const pc_params* p, const uint32_t seed[8], uint32_t kl, uint32_t* dst, hipStream_t s) {
  ExpandKeyArgs A;
  A.T = p->tabs;
  for (int w = 0; w < 8; ++w) A.key.k[w] = seed[w];
  A.dst = dst;
  A.N = (int)p->N;
  A.kl = (int)kl;
  A.L = (int)p->L;
  const dim3 grid((p->N / 8 + 255) / 256, kl + p->K, (uint32_t)beta_of(p, kl));
  LaunchTimer tm(p, KID_EXPAND_KEY, s);
  if (p->chacha_rounds == 20)
    hipLaunchKernelGGL(k_expand_key<20>, grid, dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL(k_expand_key<12>, grid, dim3(256), 0, s, A);
  return hipGetLastError();
}

#endif
}  // namespace pc
