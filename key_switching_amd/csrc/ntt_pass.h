// Two-pass negacyclic NTT for gfx950, natural order in and out.
//
// The pages name NTT kernels over the 32-bit chain (Perseus README, 'Layout')
// and leave the transform's layout open; the evaluation layout here is natural
// order, a_hat[j] = a(psi^(2j+1)).
//
// Forward (Cooley-Tukey, twiddles psi^bitrev(k)): the n = LOGRC + LOGRB stages
// split into
//   * a column pass: the first LOGRC stages only pair indices that agree mod
//     2^LOGRB, so each "column" col (elements col + 2^LOGRB * x) is an
//     independent 2^LOGRC-point problem; its twiddles are entries [1, 2^LOGRC)
//     of the table and are shared by every column;
//   * a block pass: the last LOGRB stages act inside contiguous blocks of 2^LOGRB
//     elements; block B uses entries 2^(LOGRC+s) + B 2^s + ... of the table,
//     read from a block-major copy (block B's 2^LOGRB - 1 twiddles contiguous,
//     stage s at offset 2^s); the Limb's tw of a block pass points at that copy.
// The in-place result is bit-reversed: element x of block B belongs at natural
// position bitrev(x) 2^LOGRC + bitrev(B). A workgroup therefore takes the C
// blocks B = bitrev(c0 + k), k < C, so that every output row bitrev(x) is a
// contiguous run of C words; the transpose goes through LDS.
// Inverse (Gentleman-Sande, twiddles psi^-bitrev(k)): the mirror image -- a
// block pass with the transposed load first, then a column pass.
//
// Inside a pass a workgroup holds C columns (or blocks) of R = 2^LOGR elements;
// each thread keeps E = 2^LOGE of them in registers and runs LOGE radix-2
// stages per round; rounds exchange data through LDS.  Element index held by
// thread t in round i, slot m (forward rounds walk the bits from the top,
// inverse rounds from the bottom):
//   x = (t_high << (lo + LOGE)) | (m << lo) | t_low,  t_low = t mod 2^lo.
#pragma once

#include "device_common.h"

namespace pc {

template <int LOGR, int LOGE, bool GS>
__device__ __forceinline__ int pass_lo(int round) {
  return GS ? round * LOGE : LOGR - (round + 1) * LOGE;
}

template <int LOGR, int LOGE, bool GS>
__device__ __forceinline__ int elem_index(int round, int t, int m) {
  const int lo = pass_lo<LOGR, LOGE, GS>(round);
  const int tlow = t & ((1 << lo) - 1);
  const int thigh = t >> lo;
  return (thigh << (lo + LOGE)) | (m << lo) | tlow;
}

// Row stride (words) of a column pass's LDS tile (one row per column). The
// exchanges are taken by 32 lanes of consecutive columns at a time (2 threads
// of 16 columns, or 1 of 32), writing x = 16m + t and reading x = 16t + m; for
// 256-point columns with 16 elements per thread a stride of 17 mod 32 (273)
// puts both on 32 distinct banks. Other shapes keep a pad of 4.
template <int LOGR, int LOGE = 4>
struct LdsTile {
  static constexpr int R = 1 << LOGR;
  static constexpr int STRIDE = (LOGR == 8 && LOGE == 4) ? R + 17 : R + 4;
};

// LDS layout of a block pass's tile of C blocks of R = 2^LOGRB elements:
// element x of block k at row(k) + col(x). The pass touches the tile in four
// patterns, each taken by 32 lanes at a time (32 banks of 4 bytes): two blocks
// x 16 threads writing x = 16m + t, two blocks x 16 threads reading or writing
// x = 16t + m, and 32 blocks reading or writing one x (the transpose). For
// 256-point blocks with 16 elements per thread, row(k) = 272k + k/2 and
// col(x) = x + x/16 put every one of them on 32 distinct banks (the pad makes
// 16t + m distinct over t, the stride of 16 mod 32 separates the two blocks, and
// the k/2 skew separates all 32 blocks of the transpose). 512-point blocks
// with 8 elements per thread (one block per wave) are touched as x = 64m + t,
// x = 64(t/8) + 8m + t%8 and x = 8t + m; col(x) = x + x/8 puts the last two
// on 32 distinct banks (the first has three 2-way pairs), and a row stride of
// 578 (2 mod 32) puts the two x of the 16-block transpose on even and odd
// banks. Other shapes keep a plain padded stride.
template <int LOGRB, int LOGE>
struct BlkLds {
  static constexpr int R = 1 << LOGRB;
  static constexpr bool SWZ = LOGRB == 8 && LOGE == 4;
  static constexpr bool SWZ9 = LOGRB == 9 && LOGE == 3;
  static constexpr int S = SWZ ? R + R / 16 : SWZ9 ? 578 : R + 4;
  static_assert(!SWZ9 || S >= R + R / 8, "padded row must hold x + x/8");
  __device__ __forceinline__ static int row(int k) { return SWZ ? k * S + (k >> 1) : k * S; }
  __device__ __forceinline__ static int col(int x) { return SWZ ? x + (x >> 4) : SWZ9 ? x + (x >> 3) : x; }
  static constexpr int words(int c) { return SWZ ? c * S + c / 2 : c * S; }
};

// n consecutive twiddles from p (n a power of two; p aligned to min(n, 4)
// words, which every table layout here guarantees): one vector load per four.
__device__ __forceinline__ void load_run(const uint32_t* __restrict__ p, int n, uint32_t* w) {
  if (n >= 4) {
#pragma unroll
    for (int i = 0; i < n; i += 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + i);
      w[i] = x.x;
      w[i + 1] = x.y;
      w[i + 2] = x.z;
      w[i + 3] = x.w;
    }
  } else if (n == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
    w[0] = p[0];
  }
}

// Forward CT round: stages s = round*LOGE + sl for sl < LOGE. Twiddles are in
// Montgomery form (one REDC per product). TwBase(s) returns the table offset of
// group 0 of stage s for this thread's row/block (the part that does not depend
// on the slot m); the 2^sl twiddles of stage sl are the run starting at
// TwBase(s) + (t_high << sl), indexed by m >> (LOGE - sl). FOLD0: the upper
// half of round 0 arrives already multiplied by stage 0's single twiddle.
template <int LOGR, int LOGE, bool FOLD0 = false, class TwBase>
__device__ __forceinline__ void ct_round(uint32_t (&v)[1 << LOGE], int round, int t, uint32_t r, uint32_t rinv,
                                         const uint32_t* __restrict__ tw, TwBase twbase) {
  constexpr int E = 1 << LOGE;
  const int lo = pass_lo<LOGR, LOGE, false>(round);
  const int thigh = t >> lo;
#pragma unroll
  for (int sl = 0; sl < LOGE; ++sl) {
    const int s = round * LOGE + sl;
    const int half = E >> (sl + 1);
    const bool folded = FOLD0 && s == 0;
    uint32_t w[E / 2];
    if (!folded) load_run(tw + twbase(s) + (thigh << sl), 1 << sl, w);
#pragma unroll
    for (int g = 0; g < (1 << sl); ++g) {
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const int m0 = g * 2 * half + j;
        const uint32_t u = v[m0];
        const uint32_t x = folded ? v[m0 + half] : mul_mont(v[m0 + half], w[g], r, rinv);
        v[m0] = add_mod(u, x, r);
        v[m0 + half] = sub_mod(u, x, r);
      }
    }
  }
}

// Inverse GS round: stages u = round*LOGE + ul, pairs (m, m + 2^ul). The
// 2^(LOGE-ul-1) twiddles of stage ul are the run starting at
// TwBase(u) + (t_high << (LOGE - ul - 1)), indexed by m >> (ul + 1).
template <int LOGR, int LOGE, class TwBase>
__device__ __forceinline__ void gs_round(uint32_t (&v)[1 << LOGE], int round, int t, uint32_t r, uint32_t rinv,
                                         const uint32_t* __restrict__ tw, TwBase twbase) {
  constexpr int E = 1 << LOGE;
  const int lo = pass_lo<LOGR, LOGE, true>(round);
  const int thigh = t >> lo;
#pragma unroll
  for (int ul = 0; ul < LOGE; ++ul) {
    const int u = round * LOGE + ul;
    const int half = 1 << ul;
    const int groups = E >> (ul + 1);
    uint32_t w[E / 2];
    load_run(tw + twbase(u) + (thigh << (LOGE - ul - 1)), groups, w);
#pragma unroll
    for (int g = 0; g < groups; ++g) {
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const int m0 = g * 2 * half + j;
        const uint32_t a = v[m0];
        const uint32_t b = v[m0 + half];
        v[m0] = add_mod(a, b, r);
        v[m0 + half] = mul_mont(sub_mod(a, b, r), w[g], r, rinv);
      }
    }
  }
}

// A round's twiddles gathered up front: W holds the run of every stage of the
// round (forward stage sl at [2^sl - 1, 2^(sl+1) - 1); inverse stage ul, whose
// run has E/2^(ul+1) entries, after the runs of the stages before it), so a
// pass can issue the loads of a later round before an earlier one computes.
template <int LOGR, int LOGE, bool GS, class TwBase>
__device__ __forceinline__ void load_round_tw(int round, int t, const uint32_t* __restrict__ tw, TwBase twbase,
                                              uint32_t (&W)[(1 << LOGE) - 1]) {
  constexpr int E = 1 << LOGE;
  const int lo = pass_lo<LOGR, LOGE, GS>(round);
  const int thigh = t >> lo;
  int off = 0;
#pragma unroll
  for (int st = 0; st < LOGE; ++st) {
    const int n = GS ? E >> (st + 1) : 1 << st;
    const int base = GS ? twbase(round * LOGE + st) + (thigh << (LOGE - st - 1))
                        : twbase(round * LOGE + st) + (thigh << st);
    load_run(tw + base, n, W + off);
    off += n;
  }
}

// The butterflies of ct_round / gs_round with the round's twiddles in W.
template <int LOGE>
__device__ __forceinline__ void ct_round_w(uint32_t (&v)[1 << LOGE], const uint32_t (&W)[(1 << LOGE) - 1],
                                           uint32_t r, uint32_t rinv) {
  constexpr int E = 1 << LOGE;
#pragma unroll
  for (int sl = 0; sl < LOGE; ++sl) {
    const int half = E >> (sl + 1), off = (1 << sl) - 1;
#pragma unroll
    for (int g = 0; g < (1 << sl); ++g)
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const int m0 = g * 2 * half + j;
        const uint32_t u = v[m0];
        const uint32_t x = mul_mont(v[m0 + half], W[off + g], r, rinv);
        v[m0] = add_mod(u, x, r);
        v[m0 + half] = sub_mod(u, x, r);
      }
  }
}

template <int LOGE>
__device__ __forceinline__ void gs_round_w(uint32_t (&v)[1 << LOGE], const uint32_t (&W)[(1 << LOGE) - 1],
                                           uint32_t r, uint32_t rinv) {
  constexpr int E = 1 << LOGE;
  int off = 0;
#pragma unroll
  for (int ul = 0; ul < LOGE; ++ul) {
    const int half = 1 << ul, groups = E >> (ul + 1);
#pragma unroll
    for (int g = 0; g < groups; ++g)
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const int m0 = g * 2 * half + j;
        const uint32_t a = v[m0];
        const uint32_t b = v[m0 + half];
        v[m0] = add_mod(a, b, r);
        v[m0 + half] = mul_mont(sub_mod(a, b, r), W[off + g], r, rinv);
      }
    off += groups;
  }
}

// Exchange the register tile between two round layouts through LDS; Col maps
// an element index to its word in the row.
struct IdentityCol {
  __device__ __forceinline__ static int col(int x) { return x; }
};

// Orders this wave's LDS accesses around an exchange among its own lanes: a
// wave's LDS instructions execute in program order, so only the compiler has
// to be kept from moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// WAVE: every thread that touches lds_row belongs to the calling thread's wave
// (a block pass: the 2^(LOGR-LOGE) threads of a block are consecutive lanes
// of one wave), so the exchange needs no workgroup barrier.
template <int LOGR, int LOGE, bool GS, class Col = IdentityCol, bool WAVE = false>
__device__ __forceinline__ void exchange(uint32_t (&v)[1 << LOGE], uint32_t* lds_row, int from_round, int t) {
  constexpr int E = 1 << LOGE;
#pragma unroll
  for (int m = 0; m < E; ++m) lds_row[Col::col(elem_index<LOGR, LOGE, GS>(from_round, t, m))] = v[m];
  if constexpr (WAVE)
    wave_lds_sync();
  else
    __syncthreads();
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = lds_row[Col::col(elem_index<LOGR, LOGE, GS>(from_round + 1, t, m))];
  if constexpr (WAVE)
    wave_lds_sync();
  else
    __syncthreads();
}

// The threads of one block-pass block fit in one wave (and blocks never
// straddle waves).
template <int LOGR, int LOGE>
constexpr bool block_in_wave() {
  return (1 << (LOGR - LOGE)) <= 64 && 64 % (1 << (LOGR - LOGE)) == 0;
}

// ---------------------------------------------------------------------------
// Pass bodies. A Limb policy supplies, for the limb of this workgroup:
//   r, rinv, tw                  prime, -r^-1 mod 2^32 and its twiddle table
//                                (forward or inverse, Montgomery form)
//   uint32_t load(int pos)       element at limb position pos (pass input)
//   void store(int pos, uint32_t v)  element at position pos (pass output)
// Positions are limb offsets in [0, N).
// ---------------------------------------------------------------------------

// Register-level forward column pass (the conversion kernels' transform): v
// holds this thread's E elements of column (threadIdx.x % C); the input
// layout is round 0, the output layout the last round. In round 0
// slots m and m + E/2 are stage 0's pairs (x and x + 2^(LOGRC-1)), all with
// twiddle entry 1; FOLD0: slots m >= E/2 already carry that factor.
template <int LOGRC, int LOGE, int C, bool FOLD0 = false>
__device__ __forceinline__ void fwd_col_compute(uint32_t (&v)[1 << LOGE], uint32_t* lds, uint32_t r, uint32_t rinv,
                                                const uint32_t* __restrict__ tw) {
  constexpr int ROUNDS = LOGRC / LOGE;
  const int col = threadIdx.x % C, t = threadIdx.x / C;
  auto twb = [](int s) { return 1 << s; };
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0) exchange<LOGRC, LOGE, false>(v, lds + col * LdsTile<LOGRC, LOGE>::STRIDE, rd - 1, t);
    ct_round<LOGRC, LOGE, FOLD0>(v, rd, t, r, rinv, tw, twb);
  }
}

// Limb position of slot m of this thread in a column pass: input layout (round 0)
// of a forward pass / output layout (last round) of an inverse pass.
template <int LOGRC, int LOGE, int LOGRB, int C>
__device__ __forceinline__ int col_pos_fwd_in(int col0, int m) {
  const int col = threadIdx.x % C, t = threadIdx.x / C;
  return col0 + col + (elem_index<LOGRC, LOGE, false>(0, t, m) << LOGRB);
}
template <int LOGRC, int LOGE, int LOGRB, int C>
__device__ __forceinline__ int col_pos_fwd_out(int col0, int m) {
  const int col = threadIdx.x % C, t = threadIdx.x / C;
  return col0 + col + (elem_index<LOGRC, LOGE, false>(LOGRC / LOGE - 1, t, m) << LOGRB);
}

// Register-level block passes on block B (LOGRB-point, TPB = 2^(LOGRB-LOGE)
// threads, t = this thread's index in the block, lds_row = the block's LDS row
// used for the exchanges). The forward pass takes the round-0 layout and leaves
// the last-round layout; the inverse (GS) pass likewise with its own layouts.
// Every thread of the workgroup must call these the same number of times (they
// contain barriers).
template <int LOGRC, int LOGRB, int LOGE>
__device__ __forceinline__ void fwd_blk_compute(uint32_t (&v)[1 << LOGE], uint32_t* lds_row, int t, int B,
                                                uint32_t r, uint32_t rinv, const uint32_t* __restrict__ tw) {
  constexpr int ROUNDS = LOGRB / LOGE;
  auto twb = [B](int s) { return (B << LOGRB) + (1 << s); };  // block-major table
  // every round's twiddles are requested before the first butterfly, so the
  // later rounds' loads are not waited for after the exchange
  uint32_t W[ROUNDS][(1 << LOGE) - 1];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) load_round_tw<LOGRB, LOGE, false>(rd, t, tw, twb, W[rd]);
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0)
      exchange<LOGRB, LOGE, false, BlkLds<LOGRB, LOGE>, block_in_wave<LOGRB, LOGE>()>(v, lds_row, rd - 1, t);
    ct_round_w<LOGE>(v, W[rd], r, rinv);
  }
}

template <int LOGRC, int LOGRB, int LOGE>
__device__ __forceinline__ void inv_blk_compute(uint32_t (&v)[1 << LOGE], uint32_t* lds_row, int t, int B,
                                                uint32_t r, uint32_t rinv, const uint32_t* __restrict__ tw) {
  constexpr int ROUNDS = LOGRB / LOGE;
  auto twb = [B](int u) { return (B << LOGRB) + (1 << (LOGRB - u - 1)); };  // block-major table
  uint32_t W[ROUNDS][(1 << LOGE) - 1];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) load_round_tw<LOGRB, LOGE, true>(rd, t, tw, twb, W[rd]);
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0)
      exchange<LOGRB, LOGE, true, BlkLds<LOGRB, LOGE>, block_in_wave<LOGRB, LOGE>()>(v, lds_row, rd - 1, t);
    gs_round_w<LOGE>(v, W[rd], r, rinv);
  }
}

// Forward column pass: stages 0..LOGRC-1, columns [col0, col0 + C).
template <int LOGRC, int LOGE, int LOGRB, int C, class Limb>
__device__ __forceinline__ void fwd_col_pass(Limb& L, int col0) {
  constexpr int R = 1 << LOGRC, E = 1 << LOGE, ROUNDS = LOGRC / LOGE;
  static_assert(LOGRC % LOGE == 0, "rounds must tile the pass");
  __shared__ uint32_t lds[C * LdsTile<LOGRC, LOGE>::STRIDE];
  const int tid = threadIdx.x;
  const int col = tid % C, t = tid / C;
  uint32_t v[E];
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = L.load(col0 + col + (elem_index<LOGRC, LOGE, false>(0, t, m) << LOGRB));
  auto twb = [](int s) { return 1 << s; };
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0) exchange<LOGRC, LOGE, false>(v, lds + col * LdsTile<LOGRC, LOGE>::STRIDE, rd - 1, t);
    ct_round<LOGRC, LOGE>(v, rd, t, L.r, L.rinv, L.tw, twb);
  }
#pragma unroll
  for (int m = 0; m < E; ++m)
    L.store(col0 + col + (elem_index<LOGRC, LOGE, false>(ROUNDS - 1, t, m) << LOGRB), v[m]);
  (void)R;
}

// The tile of a block pass in the segment layout: column c0 + k of the limb
// (natural positions row 2^LOGRC + c0 + k) is the contiguous run of 2^LOGRB
// words at (c0 + k) 2^LOGRB, element x (natural row bitrev(x)) at offset x.
// This is the order in which the tile sits in LDS, so consecutive lanes store
// consecutive words. Every thread of the workgroup stores E words.
template <int LOGRB, int LOGE, int C>
__device__ __forceinline__ void store_tile_segments(const uint32_t* lds, uint32_t* __restrict__ dst, int c0) {
  using Lay = BlkLds<LOGRB, LOGE>;
  constexpr int R = 1 << LOGRB, E = 1 << LOGE, THREADS = C * (R / E);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int idx = (int)threadIdx.x + THREADS * m;
    const int k = idx >> LOGRB, x = idx & (R - 1);
    at32(dst, ((c0 + k) << LOGRB) + x) = lds[Lay::row(k) + Lay::col(x)];
  }
}

// A block-pass tile of columns [c0, c0 + C) copied from natural order into the
// segment layout, through LDS.
template <int LOGRC, int LOGRB, int LOGE, int C>
__device__ __forceinline__ void copy_tile_segments(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                   int c0) {
  constexpr int R = 1 << LOGRB, E = 1 << LOGE, TPB = R / E;
  using Lay = BlkLds<LOGRB, LOGE>;
  __shared__ uint32_t lds[Lay::words(C)];
  const int kk = (int)threadIdx.x % C, rest = (int)threadIdx.x / C;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int x = rest + TPB * m;
    lds[Lay::row(kk) + Lay::col(x)] = at32(src, ((int)bitrev((uint32_t)x, LOGRB) << LOGRC) + c0 + kk);
  }
  __syncthreads();
  store_tile_segments<LOGRB, LOGE, C>(lds, dst, c0);
}

// Forward block pass: stages LOGRC..n-1 on blocks B = bitrev(c0 + k), k < C.
// Output element x of block B goes to natural position bitrev(x) 2^LOGRC + c0 + k,
// or with `seg` to the segment layout (store_tile_segments).
template <int LOGRC, int LOGRB, int LOGE, int C, class Limb>
__device__ __forceinline__ void fwd_blk_pass(Limb& L, int c0, bool seg = false) {
  constexpr int R = 1 << LOGRB, E = 1 << LOGE, ROUNDS = LOGRB / LOGE, TPB = R / E;
  static_assert(LOGRB % LOGE == 0, "rounds must tile the pass");
  using Lay = BlkLds<LOGRB, LOGE>;
  __shared__ uint32_t lds[Lay::words(C)];
  const int tid = threadIdx.x;
  const int t = tid % TPB, k = tid / TPB;
  const int B = (int)bitrev((uint32_t)(c0 + k), LOGRC);
  uint32_t v[E];
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = L.load((B << LOGRB) + elem_index<LOGRB, LOGE, false>(0, t, m));
  fwd_blk_compute<LOGRC, LOGRB, LOGE>(v, lds + Lay::row(k), t, B, L.r, L.rinv, L.tw);
  // transpose through LDS so that consecutive lanes write consecutive words
#pragma unroll
  for (int m = 0; m < E; ++m) lds[Lay::row(k) + Lay::col(elem_index<LOGRB, LOGE, false>(ROUNDS - 1, t, m))] = v[m];
  __syncthreads();
  if (seg) {
    store_tile_segments<LOGRB, LOGE, C>(lds, L.dst, c0);
    return;
  }
  const int kk = tid % C, rest = tid / C;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int x = rest + TPB * m;
    L.store(((int)bitrev((uint32_t)x, LOGRB) << LOGRC) + c0 + kk, lds[Lay::row(kk) + Lay::col(x)]);
  }
}

// Forward block pass whose output stage also reads side inputs at the output
// positions: L.fetch(m, pos) runs for every output slot m, and
// L.finish(m, pos, v) stores slot m afterwards. EARLY fetches before the
// transform, so the loads are in flight while it computes (best for small
// grids and for gathers); otherwise after it, which frees 2E registers during
// the transform and lets more workgroups share a CU (best for large grids).
template <int LOGRC, int LOGRB, int LOGE, int C, bool EARLY, class Limb>
__device__ __forceinline__ void fwd_blk_pass_fetch(Limb& L, int c0) {
  constexpr int R = 1 << LOGRB, E = 1 << LOGE, ROUNDS = LOGRB / LOGE, TPB = R / E;
  static_assert(LOGRB % LOGE == 0, "rounds must tile the pass");
  using Lay = BlkLds<LOGRB, LOGE>;
  __shared__ uint32_t lds[Lay::words(C)];
  const int tid = threadIdx.x;
  const int kk = tid % C, rest = tid / C;
  auto out_pos = [&](int m) { return ((int)bitrev((uint32_t)(rest + TPB * m), LOGRB) << LOGRC) + c0 + kk; };
  if constexpr (EARLY) {
#pragma unroll
    for (int m = 0; m < E; ++m) L.fetch(m, out_pos(m));
  }
  const int t = tid % TPB, k = tid / TPB;
  const int B = (int)bitrev((uint32_t)(c0 + k), LOGRC);
  uint32_t v[E];
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = L.load((B << LOGRB) + elem_index<LOGRB, LOGE, false>(0, t, m));
  fwd_blk_compute<LOGRC, LOGRB, LOGE>(v, lds + Lay::row(k), t, B, L.r, L.rinv, L.tw);
#pragma unroll
  for (int m = 0; m < E; ++m) lds[Lay::row(k) + Lay::col(elem_index<LOGRB, LOGE, false>(ROUNDS - 1, t, m))] = v[m];
  if constexpr (!EARLY) {
    asm volatile("" ::: "memory");  // keeps the compiler from hoisting the fetches into the transform
#pragma unroll
    for (int m = 0; m < E; ++m) L.fetch(m, out_pos(m));
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < E; ++m) L.finish(m, out_pos(m), lds[Lay::row(kk) + Lay::col(rest + TPB * m)]);
}

// Inverse block pass: GS stages 0..LOGRB-1 on blocks B = bitrev(c0 + k); element
// x of block B is read from natural position bitrev(x) 2^LOGRC + c0 + k and
// written to B 2^LOGRB + x. A non-null seg_dst also receives the input tile in
// the segment layout (store_tile_segments).
template <int LOGRC, int LOGRB, int LOGE, int C, class Limb>
__device__ __forceinline__ void inv_blk_pass(Limb& L, int c0, uint32_t* seg_dst = nullptr) {
  constexpr int R = 1 << LOGRB, E = 1 << LOGE, ROUNDS = LOGRB / LOGE, TPB = R / E;
  static_assert(LOGRB % LOGE == 0, "rounds must tile the pass");
  using Lay = BlkLds<LOGRB, LOGE>;
  __shared__ uint32_t lds[Lay::words(C)];
  const int tid = threadIdx.x;
  {
    const int kk = tid % C, rest = tid / C;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int x = rest + TPB * m;
      lds[Lay::row(kk) + Lay::col(x)] = L.load(((int)bitrev((uint32_t)x, LOGRB) << LOGRC) + c0 + kk);
    }
  }
  __syncthreads();
  if (seg_dst != nullptr) store_tile_segments<LOGRB, LOGE, C>(lds, seg_dst, c0);
  const int t = tid % TPB, k = tid / TPB;
  const int B = (int)bitrev((uint32_t)(c0 + k), LOGRC);
  uint32_t v[E];
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = lds[Lay::row(k) + Lay::col(elem_index<LOGRB, LOGE, true>(0, t, m))];
  // from here on each wave touches only its own blocks' rows, unless the
  // segment copy above read other waves' rows
  if (!block_in_wave<LOGRB, LOGE>() || seg_dst != nullptr)
    __syncthreads();
  else
    wave_lds_sync();
  inv_blk_compute<LOGRC, LOGRB, LOGE>(v, lds + Lay::row(k), t, B, L.r, L.rinv, L.tw);
#pragma unroll
  for (int m = 0; m < E; ++m) L.store((B << LOGRB) + elem_index<LOGRB, LOGE, true>(ROUNDS - 1, t, m), v[m]);
}

// Inverse column pass: GS stages LOGRB..n-1 on columns [col0, col0 + C); the
// output is in natural coefficient order (the caller's store applies N^-1).
template <int LOGRC, int LOGE, int LOGRB, int C, class Limb>
__device__ __forceinline__ void inv_col_pass(Limb& L, int col0) {
  constexpr int E = 1 << LOGE, ROUNDS = LOGRC / LOGE;
  static_assert(LOGRC % LOGE == 0, "rounds must tile the pass");
  __shared__ uint32_t lds[C * LdsTile<LOGRC, LOGE>::STRIDE];
  const int tid = threadIdx.x;
  const int col = tid % C, t = tid / C;
  uint32_t v[E];
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = L.load(col0 + col + (elem_index<LOGRC, LOGE, true>(0, t, m) << LOGRB));
  auto twb = [](int u) { return 1 << (LOGRC - u - 1); };
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0) exchange<LOGRC, LOGE, true>(v, lds + col * LdsTile<LOGRC, LOGE>::STRIDE, rd - 1, t);
    gs_round<LOGRC, LOGE>(v, rd, t, L.r, L.rinv, L.tw, twb);
  }
#pragma unroll
  for (int m = 0; m < E; ++m)
    L.store(col0 + col + (elem_index<LOGRC, LOGE, true>(ROUNDS - 1, t, m) << LOGRB), v[m]);
}

}  // namespace pc
