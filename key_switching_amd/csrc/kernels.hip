// HIP kernels for CKKS hybrid key switching on gfx950 and their launchers.
//
// Steps (Perseus README, 'Layout': NTT and key-switching kernels; 'What's
// inside': the a half regenerated in-kernel from a ChaCha12 seed):
//   ModUp   : k_modup_inv_blk + k_modup_inv_col   iNTT of c1, scaled by N^-1 (Q_d/q_i)^-1
//             k_modup_bconv_col                   fast base conversion fused into NTT pass 1
//             k_modup_fwd_blk                     NTT pass 2 -> ext (evaluation form)
//   IP      : k_inner_product                     automorphism gather, ChaCha12 a half, both sums
//   ModDown : k_md_inv_blk + k_md_inv_col         iNTT of the special limbs, scaled by N^-1 (P/p_t)^-1
//             k_md_bconv_col                      base conversion P -> q_i fused into NTT pass 1
//             k_md_fwd_blk                        NTT pass 2 fused with (acc - z) P^-1 (+ phi(c0))
// Every limb of every launch is one grid row (blockIdx.y); blockIdx.x walks the
// column/block tiles of that limb.
#include <algorithm>

#include "internal.h"
#include "ntt_pass.h"

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
  static constexpr int LRC = 8, LEC = 4, LRB = 8, LEB = 4, CC = 16, CB = 32;
};
template <>
struct Cfg<17> {
  static constexpr int LRC = 9, LEC = 3, LRB = 8, LEB = 4, CC = 16, CB = 32;
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
template <int LOGN>
constexpr int blk_tiles() {
  return (1 << Cfg<LOGN>::LRC) / Cfg<LOGN>::CB;
}

// ---------------------------------------------------------------------------
// limb policies
// ---------------------------------------------------------------------------
struct PlainLimb {
  uint32_t r;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ twp;
  const uint32_t* __restrict__ src;
  uint32_t* __restrict__ dst;
  __device__ __forceinline__ uint32_t load(int pos) const { return src[pos]; }
  __device__ __forceinline__ void store(int pos, uint32_t v) const { dst[pos] = v; }
};

struct ScaledLimb {
  uint32_t r, s, sp;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ twp;
  const uint32_t* src;
  uint32_t* dst;
  __device__ __forceinline__ uint32_t load(int pos) const { return src[pos]; }
  __device__ __forceinline__ void store(int pos, uint32_t v) const { dst[pos] = mul_shoup(v, s, sp, r); }
};

// Fast base conversion: value at pos = sum_i y_i[pos] c_i mod r, with c_i
// carrying a factor 2^32 that one REDC per pair of products removes.
struct BconvLimb {
  uint32_t r, rinv;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ twp;
  const uint32_t* __restrict__ src;  // first source limb; source k at src + k*src_stride
  size_t src_stride;
  const uint32_t* __restrict__ c;  // constant of source k at c[k * c_stride]
  int c_stride, count;
  uint32_t* __restrict__ dst;
  __device__ __forceinline__ uint32_t load(int pos) const {
    uint32_t acc = 0;
    int k = 0;
    for (; k + 1 < count; k += 2) {
      const uint64_t x = mul_wide(src[k * src_stride + pos], c[k * c_stride]) +
                         mul_wide(src[(k + 1) * src_stride + pos], c[(k + 1) * c_stride]);
      acc = add_mod(acc, redc(x, r, rinv), r);
    }
    if (k < count) acc = add_mod(acc, redc(mul_wide(src[k * src_stride + pos], c[k * c_stride]), r, rinv), r);
    return acc;
  }
  __device__ __forceinline__ void store(int pos, uint32_t v) const { dst[pos] = v; }
};

// ModDown combine: out = (acc - v) P^-1 (+ c0 at the automorphism's source index).
struct CombineLimb {
  uint32_t r, pinv, pinvp;
  const uint32_t* __restrict__ tw;
  const uint32_t* __restrict__ twp;
  const uint32_t* __restrict__ src;
  const uint32_t* __restrict__ acc;
  const uint32_t* __restrict__ c0;  // nullptr: nothing to add
  uint32_t g, h, mask;
  uint32_t* __restrict__ dst;
  __device__ __forceinline__ uint32_t load(int pos) const { return src[pos]; }
  __device__ __forceinline__ void store(int pos, uint32_t v) const {
    uint32_t o = mul_shoup(sub_mod(acc[pos], v, r), pinv, pinvp, r);
    if (c0) o = add_mod(o, c0[((uint32_t)pos * g + h) & mask], r);
    dst[pos] = o;
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
  PlainLimb L{A.T.r[pi], A.T.tw_fwd + pi * A.N, A.T.twp_fwd + pi * A.N, A.data + z * A.N, A.tmp + z * A.N};
  fwd_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_ntt_fwd_blk(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  PlainLimb L{A.T.r[pi], A.T.tw_fblk + pi * A.N, A.T.twp_fblk + pi * A.N, A.tmp + z * A.N, A.data + z * A.N};
  fwd_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_ntt_inv_blk(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  PlainLimb L{A.T.r[pi], A.T.tw_iblk + pi * A.N, A.T.twp_iblk + pi * A.N, A.data + z * A.N, A.tmp + z * A.N};
  inv_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_ntt_inv_col(NttArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, pi = A.pidx[z];
  ScaledLimb L{A.T.r[pi], A.T.ninv[pi], A.T.ninvp[pi], A.T.tw_inv + pi * A.N, A.T.twp_inv + pi * A.N,
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
  uint32_t* y;    // [batch][l][N]
  uint32_t* tmp;  // [batch][beta][l+K][N]
  uint32_t* ext;  // [batch][beta][l+K][N]
  int N, level, K, L, alpha, beta, batch, ngroups;
  size_t scale_off, bconv_off;
};

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_modup_inv_blk(ModUpArgs A) {
  using C = Cfg<LOGN>;
  // rows are prime-major (all batch items of limb i together) so that a prime's
  // twiddle slice stays in the L2 of the XCD that runs the tile
  const size_t i = blockIdx.y / A.batch, b = blockIdx.y % A.batch, z = b * A.level + i;
  PlainLimb L{A.T.r[i], A.T.tw_iblk + i * A.N, A.T.twp_iblk + i * A.N, A.ct + b * A.ct_stride + A.c1_off + i * A.N,
              A.y + z * A.N};
  inv_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_modup_inv_col(ModUpArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, i = z % A.level;
  ScaledLimb L{A.T.r[i], A.LT.mu_scale[A.scale_off + i], A.LT.mu_scalep[A.scale_off + i], A.T.tw_inv + i * A.N,
               A.T.twp_inv + i * A.N, A.y + z * A.N, A.y + z * A.N};
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

template <int G, int E, class SrcFn, class ConstFn>
__device__ __forceinline__ void grouped_bconv(TargetGroup<G, E>& tg, int cnt, SrcFn src, ConstFn cst) {
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int m = 0; m < E; ++m) tg.z[g][m] = 0;
  int k = 0;
  for (; k + 1 < cnt; k += 2) {
    uint32_t v0[E], v1[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
      v0[m] = src(k, m);
      v1[m] = src(k + 1, m);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g < tg.n) {
        const uint32_t c0 = cst(k, g), c1 = cst(k + 1, g);
#pragma unroll
        for (int m = 0; m < E; ++m)
          tg.z[g][m] = add_mod(tg.z[g][m], redc(mul_wide(v0[m], c0) + mul_wide(v1[m], c1), tg.r[g], tg.rinv[g]),
                               tg.r[g]);
      }
    }
  }
  if (k < cnt) {
    uint32_t v0[E];
#pragma unroll
    for (int m = 0; m < E; ++m) v0[m] = src(k, m);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g < tg.n) {
        const uint32_t c0 = cst(k, g);
#pragma unroll
        for (int m = 0; m < E; ++m)
          tg.z[g][m] = add_mod(tg.z[g][m], redc(mul_wide(v0[m], c0), tg.r[g], tg.rinv[g]), tg.r[g]);
      }
    }
  }
}

constexpr int kBconvGroup = 4;

// ModUp conversion: row (b, d), column tile blockIdx.x, target group blockIdx.z.
template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_modup_bconv(ModUpArgs A) {
  using C = Cfg<LOGN>;
  constexpr int E = 1 << C::LEC, G = kBconvGroup;
  __shared__ uint32_t lds[C::CC * LdsTile<C::LRC>::STRIDE];
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
  const uint32_t* ybase = A.y + (b * A.level + i0) * A.N;
  const uint32_t* cbase = A.LT.mu_bconv + A.bconv_off + (size_t)i0 * lk;
  grouped_bconv<G, E>(
      tg, cnt,
      [&](int k, int m) { return ybase[(size_t)k * A.N + col_pos_fwd_in<C::LRC, C::LEC, C::LRB, C::CC>(col0, m)]; },
      [&](int k, int g) { return cbase[(size_t)k * lk + tg.j[g]]; });
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < tg.n) {
      fwd_col_compute<C::LRC, C::LEC, C::CC>(tg.z[g], lds, tg.r[g], A.T.tw_fwd + tg.pidx[g] * A.N,
                                             A.T.twp_fwd + tg.pidx[g] * A.N);
      uint32_t* dst = A.tmp + ((b * A.beta + d) * lk + tg.j[g]) * A.N;
#pragma unroll
      for (int m = 0; m < E; ++m) dst[col_pos_fwd_out<C::LRC, C::LEC, C::LRB, C::CC>(col0, m)] = tg.z[g][m];
    }
  }
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_modup_fwd_blk(ModUpArgs A) {
  using C = Cfg<LOGN>;
  const int lk = A.level + A.K;
  const size_t nbd = (size_t)A.batch * A.beta;
  const int j = (int)(blockIdx.y / nbd);  // prime-major rows (see k_modup_inv_blk)
  const size_t bd = blockIdx.y % nbd, z = bd * lk + j;
  const int d = (int)(bd % A.beta);
  const int i0 = d * A.alpha;
  if (j >= i0 && j < min(i0 + A.alpha, A.level)) return;
  const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
  PlainLimb L{A.T.r[pj], A.T.tw_fblk + pj * A.N, A.T.twp_fblk + pj * A.N, A.tmp + z * A.N, A.ext + z * A.N};
  fwd_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

// ---------------------------------------------------------------------------
// inner product with the key: acc_u[j] = sum_d phi(ext_d[j]) * (b_d[j], a_d[j])
// Each thread owns 8 consecutive positions (one ChaCha block per digit) of limb
// j = blockIdx.y for key blockIdx.z, and loops over the batch so that the key
// values (b read, a regenerated) are loaded once per batch. Products are
// reduced with REDC in pairs; b and a are first put in Montgomery form, so the
// accumulators carry a factor 2^-64 that ModDown's constants remove.
// ---------------------------------------------------------------------------
struct IPArgs {
  DevTables T;
  const uint32_t* ct;
  uint64_t ct_stride;
  uint32_t c1_off;
  const uint32_t* ext;  // [batch][beta][l+K][N]
  uint32_t* acc;        // [items][2][l+K][N], item = key * batch + b
  int N, level, K, L, alpha, batch;
  uint32_t key_base;
  const uint32_t* evk_b[kMaxKeysPerLaunch];
  const uint32_t* evk_a[kMaxKeysPerLaunch];
  ChaChaKey seed[kMaxKeysPerLaunch];
  uint32_t galois[kMaxKeysPerLaunch];
};

constexpr int kIpThreads = 256;

// BT: the batch size when it is known at compile time (1 or 8), else 0.
template <int BETA, int ROUNDS, bool STORED, int BT>
__global__ void __launch_bounds__(kIpThreads) k_inner_product(IPArgs A) {
  const int j = blockIdx.y, key = blockIdx.z;
  const int lk = A.level + A.K;
  const int i0 = (blockIdx.x * kIpThreads + threadIdx.x) * 8;
  if (i0 >= A.N) return;
  const size_t pj = j < A.level ? (size_t)j : (size_t)(A.L + j - A.level);
  const uint32_t r = A.T.r[pj], rinv = A.T.rinv[pj];
  const uint32_t g = A.galois[key], h = (g - 1) >> 1, mask = (uint32_t)A.N - 1;

  uint32_t bm[BETA][8], am[BETA][8];
#pragma unroll
  for (int d = 0; d < BETA; ++d) {
    const uint32_t* bp = A.evk_b[key] + ((size_t)d * lk + j) * A.N + i0;
    const uint4 b0 = *reinterpret_cast<const uint4*>(bp);
    const uint4 b1 = *reinterpret_cast<const uint4*>(bp + 4);
    const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) bm[d][k] = redc(bw[k], r, rinv);
    if constexpr (STORED) {
      const uint32_t* ap = A.evk_a[key] + ((size_t)d * lk + j) * A.N + i0;
      const uint4 a0 = *reinterpret_cast<const uint4*>(ap);
      const uint4 a1 = *reinterpret_cast<const uint4*>(ap + 4);
      const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) am[d][k] = redc(aw[k], r, rinv);
    } else {
      uint32_t w[16];
      chacha_block<ROUNDS>(A.seed[key], (uint32_t)(i0 >> 3), 0u, (uint32_t)d, (uint32_t)j, w);
#pragma unroll
      for (int k = 0; k < 8; ++k) am[d][k] = word_pair_to_mont(w[2 * k], w[2 * k + 1], r, rinv);
    }
  }

  uint32_t src_idx[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) src_idx[k] = ((uint32_t)(i0 + k) * g + h) & mask;

  const int batch = BT ? BT : A.batch;
#pragma unroll 1
  for (int b = 0; b < batch; ++b) {
    uint32_t e[BETA][8];
#pragma unroll
    for (int d = 0; d < BETA; ++d) {
      const bool own = j < A.level && j >= d * A.alpha && j < (d + 1) * A.alpha;
      const uint32_t* src = own ? A.ct + b * A.ct_stride + A.c1_off + (size_t)j * A.N
                                : A.ext + (((size_t)b * BETA + d) * lk + j) * A.N;
#pragma unroll
      for (int k = 0; k < 8; ++k) e[d][k] = src[src_idx[k]];
    }
    uint32_t o0[8], o1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t s0 = 0, s1 = 0;
#pragma unroll
      for (int d = 0; d + 1 < BETA; d += 2) {
        s0 = add_mod(s0, redc(mul_wide(e[d][k], bm[d][k]) + mul_wide(e[d + 1][k], bm[d + 1][k]), r, rinv), r);
        s1 = add_mod(s1, redc(mul_wide(e[d][k], am[d][k]) + mul_wide(e[d + 1][k], am[d + 1][k]), r, rinv), r);
      }
      if constexpr (BETA % 2) {
        s0 = add_mod(s0, redc(mul_wide(e[BETA - 1][k], bm[BETA - 1][k]), r, rinv), r);
        s1 = add_mod(s1, redc(mul_wide(e[BETA - 1][k], am[BETA - 1][k]), r, rinv), r);
      }
      o0[k] = s0;
      o1[k] = s1;
    }
    const size_t item = (size_t)(A.key_base + key) * A.batch + b;
    uint32_t* a0p = A.acc + ((item * 2 + 0) * lk + j) * A.N + i0;
    uint32_t* a1p = A.acc + ((item * 2 + 1) * lk + j) * A.N + i0;
    *reinterpret_cast<uint4*>(a0p) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
    *reinterpret_cast<uint4*>(a0p + 4) = make_uint4(o0[4], o0[5], o0[6], o0[7]);
    *reinterpret_cast<uint4*>(a1p) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    *reinterpret_cast<uint4*>(a1p + 4) = make_uint4(o1[4], o1[5], o1[6], o1[7]);
  }
}

// ---------------------------------------------------------------------------
// ModDown
// ---------------------------------------------------------------------------
struct ModDownArgs {
  DevTables T;
  DevLevelTables LT;
  const uint32_t* acc;  // [items][polys][l+K][N]
  uint32_t* y2;         // [items][polys][K][N]
  uint32_t* tmp2;       // [items][polys][l][N]
  uint32_t* out;        // [items][polys][l][N]
  const uint32_t* c0;   // c0 of ciphertext b at c0 + b * ct_stride, or nullptr
  uint64_t ct_stride;
  int N, level, K, L, polys, variant, batch, rows_ip, ngroups;
  uint32_t galois[kMaxKeysPerLaunch];  // per key = item / batch
};

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_md_inv_blk(ModDownArgs A) {
  using C = Cfg<LOGN>;
  const int lk = A.level + A.K;
  // prime-major rows (see k_modup_inv_blk)
  const size_t t = blockIdx.y / A.rows_ip, ip = blockIdx.y % A.rows_ip, z = ip * A.K + t, pt = A.L + t;
  PlainLimb L{A.T.r[pt], A.T.tw_iblk + pt * A.N, A.T.twp_iblk + pt * A.N, A.acc + (ip * lk + A.level + t) * A.N,
              A.y2 + z * A.N};
  inv_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
}

template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_md_inv_col(ModDownArgs A) {
  using C = Cfg<LOGN>;
  const size_t z = blockIdx.y, t = z % A.K, pt = A.L + t;
  const size_t si = (size_t)A.variant * A.K + t;
  ScaledLimb L{A.T.r[pt], A.LT.md_scale[si], A.LT.md_scalep[si], A.T.tw_inv + pt * A.N, A.T.twp_inv + pt * A.N,
               A.y2 + z * A.N, A.y2 + z * A.N};
  inv_col_pass<C::LRC, C::LEC, C::LRB, C::CC>(L, blockIdx.x * C::CC);
}

// ModDown conversion P -> q_i: row ip = (item, u), column tile blockIdx.x,
// group of G target limbs q_i blockIdx.z.
template <int LOGN>
__global__ void __launch_bounds__(col_threads<LOGN>()) k_md_bconv(ModDownArgs A) {
  using C = Cfg<LOGN>;
  constexpr int E = 1 << C::LEC, G = kBconvGroup;
  __shared__ uint32_t lds[C::CC * LdsTile<C::LRC>::STRIDE];
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
  const uint32_t* ybase = A.y2 + ip * A.K * A.N;
  const uint32_t* cbase = A.LT.md_bconv + (size_t)A.variant * A.K * A.L;
  grouped_bconv<G, E>(
      tg, A.K,
      [&](int k, int m) { return ybase[(size_t)k * A.N + col_pos_fwd_in<C::LRC, C::LEC, C::LRB, C::CC>(col0, m)]; },
      [&](int k, int g) { return cbase[(size_t)k * A.L + tg.j[g]]; });
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < tg.n) {
      fwd_col_compute<C::LRC, C::LEC, C::CC>(tg.z[g], lds, tg.r[g], A.T.tw_fwd + tg.pidx[g] * A.N,
                                             A.T.twp_fwd + tg.pidx[g] * A.N);
      uint32_t* dst = A.tmp2 + (ip * A.level + tg.j[g]) * A.N;
#pragma unroll
      for (int m = 0; m < E; ++m) dst[col_pos_fwd_out<C::LRC, C::LEC, C::LRB, C::CC>(col0, m)] = tg.z[g][m];
    }
  }
}

template <int LOGN>
__global__ void __launch_bounds__(blk_threads<LOGN>()) k_md_fwd_blk(ModDownArgs A) {
  using C = Cfg<LOGN>;
  const int lk = A.level + A.K;
  // prime-major rows (see k_modup_inv_blk)
  const size_t i = blockIdx.y / A.rows_ip, ip = blockIdx.y % A.rows_ip, z = ip * A.level + i;
  const size_t item = ip / A.polys, u = ip % A.polys;
  const size_t pi = (size_t)A.variant * A.L + i;
  const uint32_t* c0 = nullptr;
  uint32_t g = 1;
  if (A.c0 != nullptr && u == 0) {
    c0 = A.c0 + (item % A.batch) * A.ct_stride + i * A.N;
    g = A.galois[item / A.batch];
  }
  CombineLimb L{A.T.r[i],
                A.LT.md_pinv[pi],
                A.LT.md_pinvp[pi],
                A.T.tw_fblk + i * A.N,
                A.T.twp_fblk + i * A.N,
                A.tmp2 + z * A.N,
                A.acc + (ip * lk + i) * A.N,
                c0,
                g,
                (g - 1) >> 1,
                (uint32_t)A.N - 1,
                A.out + z * A.N};
  fwd_blk_pass<C::LRC, C::LRB, C::LEB, C::CB>(L, blockIdx.x * C::CB);
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

static int alpha_at(const pc_params* p, uint32_t level) { return (int)((level + p->dnum - 1) / p->dnum); }
static int beta_at(const pc_params* p, uint32_t level) {
  const int a = alpha_at(p, level);
  return (int)((level + a - 1) / a);
}

hipError_t launch_modup(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset, uint32_t batch,
                        uint32_t level, const KsWorkspace& ws, hipStream_t s) {
  ModUpArgs A;
  A.T = p->tabs;
  A.LT = p->ltabs;
  A.ct = ct;
  A.ct_stride = ct_stride;
  A.c1_off = c1_offset;
  A.y = ws.y;
  A.tmp = ws.tmp;
  A.ext = ws.ext;
  A.N = (int)p->N;
  A.level = (int)level;
  A.K = (int)p->K;
  A.L = (int)p->L;
  A.alpha = alpha_at(p, level);
  A.beta = beta_at(p, level);
  A.scale_off = p->mu_scale_off[level];
  A.bconv_off = p->mu_bconv_off[level];
  A.batch = (int)batch;
  const uint32_t rows_in = batch * level;
  const uint32_t rows_ext = batch * (uint32_t)A.beta * (level + p->K);
  // the last digit is the shortest, so it has the most targets
  const int targets = (int)(level + p->K) - ((int)level - (A.beta - 1) * A.alpha);
  const uint32_t groups = (uint32_t)((targets + kBconvGroup - 1) / kBconvGroup);
  A.ngroups = (int)groups;
  PC_DISPATCH_LOGN(p->log2n, {
    { LaunchTimer tm(p, KID_MODUP_INV_BLK, s); hipLaunchKernelGGL(k_modup_inv_blk<LN>, dim3(blk_tiles<LN>(), rows_in), dim3(blk_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODUP_INV_COL, s); hipLaunchKernelGGL(k_modup_inv_col<LN>, dim3(col_tiles<LN>(), rows_in), dim3(col_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODUP_BCONV, s); hipLaunchKernelGGL(k_modup_bconv<LN>, dim3(xcd_grid(col_tiles<LN>(), (int)batch * A.beta, (int)groups)), dim3(col_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODUP_FWD_BLK, s); hipLaunchKernelGGL(k_modup_fwd_blk<LN>, dim3(blk_tiles<LN>(), rows_ext), dim3(blk_threads<LN>()), 0, s, A); }
  });
  return hipGetLastError();
}

template <int BETA, int BT>
static void launch_ip_bt(const pc_params* p, const IPArgs& A, uint32_t nkeys, bool stored, hipStream_t s) {
  const dim3 grid((p->N / 8 + kIpThreads - 1) / kIpThreads, (uint32_t)(A.level + A.K), nkeys);
  LaunchTimer tm(p, KID_INNER_PRODUCT, s);
  if (stored)
    hipLaunchKernelGGL((k_inner_product<BETA, 12, true, BT>), grid, dim3(kIpThreads), 0, s, A);
  else if (p->chacha_rounds == 20)
    hipLaunchKernelGGL((k_inner_product<BETA, 20, false, BT>), grid, dim3(kIpThreads), 0, s, A);
  else
    hipLaunchKernelGGL((k_inner_product<BETA, 12, false, BT>), grid, dim3(kIpThreads), 0, s, A);
}

template <int BETA>
static void launch_ip_beta(const pc_params* p, const IPArgs& A, uint32_t nkeys, bool stored, hipStream_t s) {
  if (A.batch == 8)
    launch_ip_bt<BETA, 8>(p, A, nkeys, stored, s);
  else if (A.batch == 1)
    launch_ip_bt<BETA, 1>(p, A, nkeys, stored, s);
  else
    launch_ip_bt<BETA, 0>(p, A, nkeys, stored, s);
}

hipError_t launch_inner_product(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset,
                                uint32_t batch, uint32_t level, const KsWorkspace& ws, const KeyRef* keys,
                                uint32_t nkeys, hipStream_t s) {
  const int beta = beta_at(p, level);
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
    A.alpha = alpha_at(p, level);
    A.batch = (int)batch;
    A.key_base = base;
    bool stored = false;
    for (uint32_t k = 0; k < cnt; ++k) {
      const KeyRef& kr = keys[base + k];
      A.evk_b[k] = kr.b;
      A.evk_a[k] = kr.a;
      stored = stored || kr.a != nullptr;
      for (int w = 0; w < 8; ++w) A.seed[k].k[w] = kr.seed[w];
      A.galois[k] = kr.galois;
    }
    switch (beta) {
      case 1: launch_ip_beta<1>(p, A, cnt, stored, s); break;
      case 2: launch_ip_beta<2>(p, A, cnt, stored, s); break;
      case 3: launch_ip_beta<3>(p, A, cnt, stored, s); break;
      case 4: launch_ip_beta<4>(p, A, cnt, stored, s); break;
      case 5: launch_ip_beta<5>(p, A, cnt, stored, s); break;
      case 6: launch_ip_beta<6>(p, A, cnt, stored, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_moddown(const pc_params* p, const uint32_t* acc, uint32_t items, uint32_t polys, uint32_t level,
                          int variant, uint32_t* out, const KsWorkspace& ws, const uint32_t* c0, uint64_t ct_stride,
                          uint32_t batch, const uint32_t* galois_per_key, hipStream_t s) {
  ModDownArgs A;
  A.T = p->tabs;
  A.LT = p->ltabs;
  A.acc = acc;
  A.y2 = ws.y2;
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
  const uint32_t rows_q = items * polys * level;
  const uint32_t groups = (level + kBconvGroup - 1) / kBconvGroup;
  A.rows_ip = (int)(items * polys);
  A.ngroups = (int)groups;
  PC_DISPATCH_LOGN(p->log2n, {
    { LaunchTimer tm(p, KID_MODDOWN_INV_BLK, s); hipLaunchKernelGGL(k_md_inv_blk<LN>, dim3(blk_tiles<LN>(), rows_p), dim3(blk_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODDOWN_INV_COL, s); hipLaunchKernelGGL(k_md_inv_col<LN>, dim3(col_tiles<LN>(), rows_p), dim3(col_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODDOWN_BCONV, s); hipLaunchKernelGGL(k_md_bconv<LN>, dim3(xcd_grid(col_tiles<LN>(), (int)(items * polys), (int)groups)), dim3(col_threads<LN>()), 0, s, A); }
    { LaunchTimer tm(p, KID_MODDOWN_FWD_BLK, s); hipLaunchKernelGGL(k_md_fwd_blk<LN>, dim3(blk_tiles<LN>(), rows_q), dim3(blk_threads<LN>()), 0, s, A); }
  });
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

}  // namespace pc
