// Internal types shared by the C-ABI layer (capi.hip) and the kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/pc.h"

namespace pc {

constexpr int kMaxLimbsPerLaunch = 256;  // prime indices travel in kernel arguments
constexpr int kMaxKeysPerLaunch = 32;    // keys (seeds, pointers, Galois elements) per inner-product launch
constexpr int kMaxDigits = 6;            // digits supported by the inner-product kernel
constexpr int kMaxSpecial = 8;           // special primes (ModDown)
constexpr int kMaxAlpha = 8;             // primes per digit (ModUp)
constexpr int kMaxRescaleLimbs = 64;     // limbs kept by a rescale (constants travel in kernel arguments)
// Words between consecutive limbs of the inverse passes' buffers (ModUp's y,
// ModDown's y2) beyond N: with limbs a power of two apart, the workgroups
// that walk many limbs at the same offsets meet on the same HBM channels.
constexpr uint32_t kLimbPad = 32;

// Device pointers to the per-prime tables (prime index = position in the chain:
// q_0..q_{L-1} then p_0..p_{K-1}).
struct DevTables {
  const uint32_t* r;        // [P] primes
  const uint32_t* rinv;     // [P] -r^-1 mod 2^32
  const uint32_t* ninv;     // [P] N^-1 mod r
  const uint32_t* ninvp;    // [P] Shoup companions
  const uint32_t* r2;       // [P] 2^64 mod r (leaves Montgomery form through one REDC)
  // twiddles in Montgomery form (w 2^32 mod r), so that one REDC of x*w gives x*w mod r
  const uint32_t* tw_fwd;   // [P][N] psi^bitrev(k)
  const uint32_t* tw_inv;   // [P][N] psi^-bitrev(k)
  // block-major copies for the block passes: block B's twiddles are the run
  // [B 2^LRB + 1, B 2^LRB + 2^LRB), stage s of the forward pass at offset 2^s,
  // stage u of the inverse pass at offset 2^(LRB-u-1) (each stage's run is
  // aligned to its length)
  const uint32_t* tw_fblk;  // [P][N]
  const uint32_t* tw_iblk;  // [P][N]
};

// Split of the n = log2 N NTT stages into a column pass of 2^lrc points and a
// block pass of 2^lrb points (must match the kernels' pass shapes).
constexpr int pass_split_lrc(uint32_t log2n) { return log2n == 12 ? 6 : log2n == 16 ? 8 : log2n == 17 ? 8 : -1; }
inline bool pass_split(uint32_t log2n, int* lrc, int* lrb) {
  const int c = pass_split_lrc(log2n);
  if (c < 0) return false;
  *lrc = c;
  *lrb = (int)log2n - c;
  return true;
}

// Per-level constants for ModUp and ModDown (level l = number of active q primes).
struct DevLevelTables {
  const uint32_t* mu_scale;   // [sum_l l] N^-1 (Q_d/q_i)^-1 mod q_i, by level then limb
  const uint32_t* mu_scalep;
  const uint32_t* mu_bconv;   // [sum_l l (l+K)] (Q_d/q_i) 2^32 mod r_j, by level, source limb i, target j
  // ModDown, two variants v: 0 = plain input, 1 = input carrying a factor 2^-64
  const uint32_t* md_scale;   // [2][K] N^-1 (P/p_t)^-1 S mod p_t
  const uint32_t* md_scalep;
  const uint32_t* md_bconv;   // [2][K][L] (P/p_t) 2^32 S^-1 mod q_i
  const uint32_t* md_pinv;    // [2][L] S P^-1 mod q_i
  const uint32_t* md_pinvp;
  // the conversion constants times the target's first forward twiddle
  // psi^bitrev(1) (plain): the upper half of a column, which the NTT's first
  // stage multiplies by that twiddle, is converted already multiplied by it
  const uint32_t* mu_bconvw;  // as mu_bconv
  const uint32_t* md_bconvw;  // as md_bconv
};

}  // namespace pc

struct pc_params {
  int device = -1;
  uint32_t log2n = 0, N = 0, L = 0, dnum = 0, K = 0;
  uint32_t max_batch = 1, max_hoist = 1, chacha_rounds = 12, partition = 0;
  std::vector<uint32_t> primes;  // L q-primes then K p-primes
  std::vector<uint32_t> psi;
  // host copies of the tables (always built; uploaded when device >= 0)
  std::vector<uint32_t> h_rinv, h_ninv, h_ninvp, h_r2;
  std::vector<uint32_t> h_tw_fwd, h_tw_inv;                       // psi^+-bitrev(k), plain
  std::vector<uint32_t> h_twm_fwd, h_twm_inv, h_twm_fblk, h_twm_iblk;  // Montgomery form, uploaded
  std::vector<uint32_t> h_mu_scale, h_mu_scalep, h_mu_bconv;
  std::vector<size_t> mu_scale_off, mu_bconv_off;  // by level (index l, 1..L)
  std::vector<uint32_t> h_md_scale, h_md_scalep, h_md_bconv, h_md_pinv, h_md_pinvp;
  std::vector<uint32_t> h_mu_bconvw, h_md_bconvw;  // the conversion constants times psi^bitrev(1) of the target
  // rescale by q_{l'} (row l' = level - 1, entry i < l'): q_{l'} mod q_i, q_{l'}^-1 mod q_i, its Shoup companion
  std::vector<uint32_t> h_rs_qlmod, h_rs_inv, h_rs_invp;  // [L][L]
  // device state
  void* d_tables = nullptr;  // one allocation holding every table
  pc::DevTables tabs{};
  pc::DevLevelTables ltabs{};
  void* arena = nullptr;  // workspace arena sized at create
  size_t arena_bytes = 0;
  // measurement support (pc_profile_begin / pc_profile_end)
  mutable bool prof_on = false;
  mutable std::vector<hipEvent_t> prof_pool;  // events owned by the params
  mutable size_t prof_used = 0;               // events handed out in this window
  struct ProfRec {
    int kernel;
    hipEvent_t start, stop;
  };
  mutable std::vector<ProfRec> prof_recs;
};

// A key bundle (pc_keyset): nkeys keys of one key level in one device
// allocation, each key's b half and, in the FULL mode, its expanded a half.
struct pc_keyset {
  const pc_params* p = nullptr;
  uint32_t key_level = 0, nkeys = 0, mode = 0, beta = 0, lk = 0;
  size_t key_words = 0;          // beta * lk * N: one key half
  uint32_t* mem = nullptr;       // [nkeys][halves][beta][lk][N], halves = 1 (b) or 2 (b, a)
  std::vector<uint32_t> galois;  // [nkeys]
  std::vector<uint8_t> seeds;    // [nkeys][32]
  uint32_t* b_of(uint32_t k) const { return mem + (size_t)k * (mode ? 2 : 1) * key_words; }
  uint32_t* a_of(uint32_t k) const { return mode ? mem + ((size_t)k * 2 + 1) * key_words : nullptr; }
};

namespace pc {

// Digit size and count at a level, and the level of the key that serves it
// (partition 0: ceil(l/dnum) and l; partition 1: ceil(L/dnum) and L).
inline int alpha_of(const pc_params* p, uint32_t level) {
  const uint32_t l = p->partition ? p->L : level;
  return (int)((l + p->dnum - 1) / p->dnum);
}
inline int beta_of(const pc_params* p, uint32_t level) {
  const int a = alpha_of(p, level);
  return (int)((level + a - 1) / a);
}
inline uint32_t key_level_of(const pc_params* p, uint32_t level) { return p->partition ? p->L : level; }

// Workspace carve-up for a key switch of `items` (ciphertext, key) pairs over a
// batch of `batch` ciphertexts at level l.
struct KsWorkspace {
  uint32_t* y;     // [batch][l][N + kLimbPad] ModUp coefficients (scaled)
  uint32_t* tmp;   // [batch][beta][l+K][N]  ModUp after the column pass
  uint32_t* ext;   // [batch][beta][l+K][N]  ModUp output (evaluation form)
  uint32_t* acc;   // [items][2][l+K][N]     inner product
  uint32_t* y2;    // [items][2][K][N + kLimbPad] ModDown coefficients of the P limbs
  uint32_t* tmp2;  // [items][2][l][N]       ModDown after the column pass
  // ext in the segment layout, for inner products that gather under
  // automorphisms (set before ModUp; ModUp then also files c1's limbs there)
  bool seg = false;
};
size_t ks_workspace_bytes(const pc_params* p, uint32_t level, uint32_t batch, uint32_t items);
KsWorkspace ks_workspace_carve(const pc_params* p, void* base, uint32_t level, uint32_t batch, uint32_t items);

struct KeyRef {
  const uint32_t* b;  // [beta][l+K][N]
  const uint32_t* a;  // stored a half (same shape) or nullptr to regenerate from seed
  uint32_t seed[8];
  uint32_t galois;
};

// Kernel families for measurement (names in kKernelNames).
enum KernelId {
  KID_NTT_FWD_COL,
  KID_NTT_FWD_BLK,
  KID_NTT_INV_BLK,
  KID_NTT_INV_COL,
  KID_MODUP_INV_BLK,
  KID_MODUP_INV_COL,
  KID_MODUP_BCONV,
  KID_MODUP_FWD_BLK,
  KID_INNER_PRODUCT,
  KID_MODDOWN_INV_BLK,
  KID_MODDOWN_INV_COL,
  KID_MODDOWN_BCONV,
  KID_MODDOWN_FWD_BLK,
  KID_CHACHA_EXPAND,
  KID_KEYGEN,
  KID_TENSOR,
  KID_RESCALE_GATHER,
  KID_RESCALE_COL,
  KID_RESCALE_BLK,
  KID_BSGS_BABY,
  KID_BSGS_GIANT,
  KID_SEG_COPY,
  KID_MODDOWN_RESCALE,
  KID_EXPAND_KEY,
  KID_MODUP_IP,
  KID_COUNT
};
extern const char* const kKernelNames[KID_COUNT];

// Brackets one launch with events when profiling is on (no-op otherwise).
struct LaunchTimer {
  const pc_params* p;
  int kernel;
  hipStream_t s;
  hipEvent_t start = nullptr;
  LaunchTimer(const pc_params* params, int kid, hipStream_t stream);
  ~LaunchTimer();
};

// Launchers (return hipError_t of the last launch).
hipError_t launch_ntt(const pc_params* p, uint32_t* data, uint32_t* tmp, const uint32_t* prime_idx, uint32_t nlimbs,
                      bool inverse, hipStream_t s);
// fwd_blk = false stops after the conversion's column pass (tmp), for the fused
// block pass and inner product.
hipError_t launch_modup(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset, uint32_t batch,
                        uint32_t level, const KsWorkspace& ws, hipStream_t s, bool fwd_blk = true);
// ModUp and the inner product of `batch` ciphertexts under `nkeys` keys (every
// key on the same batch). One key of Galois element 1 takes the fused block
// pass and inner product (no ext round trip through memory) when its key tile
// fits a thread's budget; other calls run ModUp to ext and the inner product.
hipError_t launch_modup_ip(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset,
                           uint32_t batch, uint32_t level, const KsWorkspace& ws, const KeyRef* keys, uint32_t nkeys,
                           hipStream_t s);
// one_ct_per_key: key k switches its own `batch` ciphertexts, the k-th group
// (ct + k batch ct_stride, ext of ModUp's items k batch .. k batch + batch - 1);
// otherwise every key switches the same batch.
hipError_t launch_inner_product(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_offset,
                                uint32_t batch, uint32_t level, const KsWorkspace& ws, const KeyRef* keys,
                                uint32_t nkeys, hipStream_t s, bool one_ct_per_key = false);
// ModDown of items*2 accumulators; out[item][u][l][N]. variant: 0 plain acc, 1 acc carrying 2^-64.
// When c0 is non-null, c0 of ciphertext (item % batch) under the item's Galois element is added to u = 0.
hipError_t launch_moddown(const pc_params* p, const uint32_t* acc, uint32_t items, uint32_t polys, uint32_t level,
                          int variant, uint32_t* out, const KsWorkspace& ws, const uint32_t* c0, uint64_t ct_stride,
                          uint32_t batch, const uint32_t* galois_per_key, hipStream_t s, bool c0_seg = false,
                          uint32_t combine_from = 0);
// Copy of `limbs` limbs from natural order into the segment layout (dst must not overlap src).
hipError_t launch_seg_copy(const pc_params* p, const uint32_t* src, uint32_t limbs, uint32_t* dst, hipStream_t s);
// b of a key at `level` from evaluation-form s ([lk][N]) and e ([beta][lk][N]);
// gm[j] = [P]_{q_j} 2^32 mod q_j (q-limbs).
hipError_t launch_keygen(const pc_params* p, const uint32_t seed[8], uint32_t level, uint32_t galois,
                         const uint32_t* s_eval, const uint32_t* e_eval, const uint32_t* gm, uint32_t* evk_b,
                         hipStream_t s);
// Tensor product of `batch` ciphertext pairs at `level` (evaluation form):
// pair z reads a + z a_stride and b + z b_stride ([2][l][N] each) and writes
// d_k at d + z d_stride + d_off[k] ([l][N]) for d0 = a0 b0, d1 = a0 b1 + a1 b0,
// d2 = a1 b1.
hipError_t launch_tensor(const pc_params* p, const uint32_t* a, uint64_t a_stride, const uint32_t* b,
                         uint64_t b_stride, uint32_t batch, uint32_t level, uint32_t* d, uint64_t d_stride,
                         const uint64_t d_off[3], hipStream_t s);
// Rescale of `batch` ciphertexts at `level` by their last prime: polynomial v
// of ciphertext b at c + b c_stride + v c1_off ([l][N]); when add1 is non-null,
// add1 + b add_stride ([l][N]) is added to polynomial 1 first. x ([2 batch][N])
// and tmp ([2 batch][l-1][N]) are workspace; out is [batch][2][l-1][N].
hipError_t launch_rescale(const pc_params* p, const uint32_t* c, uint64_t c_stride, uint32_t c1_off,
                          const uint32_t* add1, uint64_t add_stride, uint32_t batch, uint32_t level, uint32_t* x,
                          uint32_t* tmp, uint32_t* out, hipStream_t s, bool final_pass = true);
// The ModDown combine of limbs 0..level-2 of a relinearised batch fused with the
// rescale's last pass: launch_moddown(..., combine_from = level - 1) has
// written limb level-1 and launch_rescale(..., final_pass = false) has filled
// tmp; out = [batch][2][level-1][N]. c0 and add1 as in launch_moddown and
// launch_rescale (d0 and d1 of the tensor).
hipError_t launch_moddown_rescale(const pc_params* p, const uint32_t* acc, uint32_t batch, uint32_t level,
                                  const KsWorkspace& ws, const uint32_t* c0, uint64_t ct_stride,
                                  const uint32_t* add1, uint64_t add_stride, const uint32_t* tmp, uint32_t* out,
                                  hipStream_t s);
// Baby steps of the double-hoisted linear transform: inner [2][n2][l+K][N] from
// the ciphertext [2][l][N], the baby inner products acc [n1-1][2][l+K][N] (factor
// 2^-64) and the diagonals [n2][n1][l+K][N]; per extended-basis limb t:
// pm = P 2^64 mod r_t (q-limbs), m96 = 2^96 mod r_t, m128 = 2^128 mod r_t.
hipError_t launch_bsgs_baby(const pc_params* p, const uint32_t* ct, const uint32_t* acc, const uint32_t* diag,
                            uint32_t* inner, uint32_t level, uint32_t n1, uint32_t n2, const uint32_t* baby_galois,
                            const uint32_t* pm, const uint32_t* m96, const uint32_t* m128, hipStream_t s);
// Giant-step sum: accqp [2][l+K][N] = inner_0 + sum_{j>=1} (phi_{G_j}(inner_j,0), 0) + 2^64 accg_j.
hipError_t launch_bsgs_giant(const pc_params* p, const uint32_t* inner, const uint32_t* accg, uint32_t* accqp,
                             uint32_t level, uint32_t n2, const uint32_t* giant_galois, const uint32_t* pm,
                             const uint32_t* m96, const uint32_t* m128, hipStream_t s);
hipError_t launch_chacha_expand(const pc_params* p, const uint32_t seed[8], uint32_t d, uint32_t j,
                                uint32_t prime_index, uint32_t* dst, hipStream_t s);
// Every limb of a key's a half at key level kl: dst [beta][kl+K][N], canonical.
hipError_t launch_expand_key(const pc_params* p, const uint32_t seed[8], uint32_t kl, uint32_t* dst, hipStream_t s);

}  // namespace pc
