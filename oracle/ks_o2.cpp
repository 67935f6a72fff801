// Second oracle tier: RNS-CKKS hybrid key switching in plain C++17, OpenMP over
// independent (digit, limb) items. Test infrastructure only: the tests and the
// benchmark's CPU baseline load it; the GPU library never does. It shares no
// code, header or table with the GPU library or with the numpy oracle: it
// finds its own primes and roots; every modular product is the plain
// (uint64)a*b % r, sums and differences a conditional correction.
//
// Source of the method: the Perseus README ('What's inside': one half of each
// key-switching key is re-created from a ChaCha12 seed on the device;
// 'Layout': the NTT and key-switching kernels) and the arXiv summary page of
// the Perseus paper (methodology item (i): ChaCha12 in counter mode). The
// pages do not write hybrid key switching out; this follows the textbook RNS
// algorithm with fast base conversion, under the same readings as the numpy
// oracle:
//   * primes: every q = 1 mod 2N below 2^31, largest first (trial division);
//     q_0..q_{L-1} then p_0..p_{K-1};
//   * psi: the smallest x >= 2 with x^N = -1 mod r (search from 2 upward);
//   * evaluation form in natural order: a_hat[j] = sum_i a_i psi^((2j+1)i);
//   * digits: alpha = ceil(l/dnum) primes each (partition 0, key at level l)
//     or ceil(L/dnum) at every level (partition 1, one key at level L);
//   * key limb j of the extended basis: j for q limbs, key level + (j - l)
//     for the special primes; the a half's limb (d, j) is the ChaCha stream
//     with nonce (0, d, key limb), value i = (w[2i] + 2^32 w[2i+1]) mod r;
//   * automorphism X -> X^k in evaluation form: out[i] = in[(i k + (k-1)/2) mod N];
//   * ModDown in floor form: (acc - Conv_{P->Q}([acc]_P)) * P^-1.
//
// Build: g++ -O2 -std=c++17 -fopenmp -shared -fPIC ks_o2.cpp -o libks_o2.so
#include <omp.h>

#include <cstdint>
#include <cstring>
#include <vector>

namespace {

using u32 = uint32_t;
using u64 = uint64_t;

// a * b mod r for any 32-bit a, b; a + b and a - b for canonical a, b < r.
u32 mulm(u32 a, u32 b, u32 r) { return (u32)((u64)a * b % r); }
u32 addm(u32 a, u32 b, u32 r) {
  const u64 s = (u64)a + b;
  return (u32)(s >= r ? s - r : s);
}
u32 subm(u32 a, u32 b, u32 r) { return a >= b ? a - b : a + (r - b); }

u32 powm(u32 a, u64 e, u32 r) {
  u64 x = a % r, y = 1;
  while (e) {
    if (e & 1) y = y * x % r;
    x = x * x % r;
    e >>= 1;
  }
  return (u32)y;
}

// a^-1 mod r for prime r (Fermat).
u32 invm(u32 a, u32 r) { return powm(a, r - 2, r); }

bool is_prime(u32 n) {
  if (n < 2) return false;
  for (u32 d = 2; (u64)d * d <= n; ++d)
    if (n % d == 0) return false;
  return true;
}

// The `count` largest primes below 2^31 that are 1 mod 2N, largest first.
std::vector<u32> prime_chain(u32 N, int count) {
  std::vector<u32> out;
  const u64 m = 2ull * N;
  for (u64 c = (1ull << 31) - m + 1; c > m && (int)out.size() < count; c -= m)
    if (is_prime((u32)c)) out.push_back((u32)c);
  return out;
}

u32 smallest_psi(u32 r, u32 N) {
  for (u32 x = 2; x < r; ++x)
    if (powm(x, N, r) == r - 1) return x;
  return 0;
}

u32 bit_reverse(u32 x, int bits) {
  u32 y = 0;
  for (int i = 0; i < bits; ++i) y |= ((x >> i) & 1u) << (bits - 1 - i);
  return y;
}

// Negacyclic NTT for one prime: a pre-twist by psi^i, then a cyclic DFT with
// omega = psi^2, so that psi^i omega^(ij) = psi^((2j+1)i).
struct Ntt {
  u32 r = 0, N = 0, psi = 0, psi_inv = 0, n_inv = 0;
  int logn = 0;
  std::vector<u32> pw, pw_inv;  // psi^i, psi^-i

  void init(u32 r_, u32 N_, int logn_) {
    r = r_;
    N = N_;
    logn = logn_;
    psi = smallest_psi(r, N);
    psi_inv = invm(psi, r);
    pw.resize(N);
    pw_inv.resize(N);
    pw[0] = pw_inv[0] = 1;
    for (u32 i = 1; i < N; ++i) {
      pw[i] = mulm(pw[i - 1], psi, r);
      pw_inv[i] = mulm(pw_inv[i - 1], psi_inv, r);
    }
    n_inv = invm(N % r, r);
  }

  // x[j] <- sum_i x[i] w^(ij), w of order N: bit-reversal permutation, then
  // iterative radix-2 decimation in time.
  void cyclic(u32* x, u32 w) const {
    for (u32 i = 0; i < N; ++i) {
      const u32 j = bit_reverse(i, logn);
      if (i < j) {
        const u32 t = x[i];
        x[i] = x[j];
        x[j] = t;
      }
    }
    for (u32 len = 2; len <= N; len <<= 1) {
      const u32 h = len / 2, wl = powm(w, N / len, r);
      for (u32 s = 0; s < N; s += len) {
        u32 wk = 1;
        for (u32 k = 0; k < h; ++k) {
          const u32 u = x[s + k], v = mulm(x[s + k + h], wk, r);
          x[s + k] = addm(u, v, r);
          x[s + k + h] = subm(u, v, r);
          wk = mulm(wk, wl, r);
        }
      }
    }
  }

  void forward(u32* x) const {
    for (u32 i = 0; i < N; ++i) x[i] = mulm(x[i], pw[i], r);
    cyclic(x, mulm(psi, psi, r));
  }

  // a[i] = N^-1 psi^-i sum_j a_hat[j] omega^(-ij)
  void inverse(u32* x) const {
    cyclic(x, mulm(psi_inv, psi_inv, r));
    for (u32 i = 0; i < N; ++i) x[i] = mulm(mulm(x[i], pw_inv[i], r), n_inv, r);
  }
};

u32 rotl(u32 v, int n) { return (v << n) | (v >> (32 - n)); }

void quarter(u32* x, int a, int b, int c, int d) {
  x[a] += x[b]; x[d] = rotl(x[d] ^ x[a], 16);
  x[c] += x[d]; x[b] = rotl(x[b] ^ x[c], 12);
  x[a] += x[b]; x[d] = rotl(x[d] ^ x[a], 8);
  x[c] += x[d]; x[b] = rotl(x[b] ^ x[c], 7);
}

// One ChaCha block in the RFC 8439 state layout (constants, 8 key words, the
// block counter, 3 nonce words); `rounds` rounds alternating column and
// diagonal rounds; output = final state + initial state.
void chacha_block(const u32 key[8], u32 counter, const u32 nonce[3], int rounds, u32 out[16]) {
  u32 s[16] = {0x61707865u, 0x3320646eu, 0x79622d32u, 0x6b206574u};
  for (int i = 0; i < 8; ++i) s[4 + i] = key[i];
  s[12] = counter;
  s[13] = nonce[0];
  s[14] = nonce[1];
  s[15] = nonce[2];
  u32 x[16];
  std::memcpy(x, s, sizeof x);
  for (int i = 0; i < rounds; i += 2) {
    quarter(x, 0, 4, 8, 12);
    quarter(x, 1, 5, 9, 13);
    quarter(x, 2, 6, 10, 14);
    quarter(x, 3, 7, 11, 15);
    quarter(x, 0, 5, 10, 15);
    quarter(x, 1, 6, 11, 12);
    quarter(x, 2, 7, 8, 13);
    quarter(x, 3, 4, 9, 14);
  }
  for (int i = 0; i < 16; ++i) out[i] = x[i] + s[i];
}

struct Ctx {
  int logn = 0, L = 0, dnum = 0, K = 0, partition = 0, rounds = 12;
  u32 N = 0;
  std::vector<u32> primes;  // q_0..q_{L-1}, p_0..p_{K-1}
  std::vector<Ntt> ntt;     // one per prime

  int alpha(int level) const { return ((partition ? L : level) + dnum - 1) / dnum; }
  int key_level(int level) const { return partition ? L : level; }
  // index into `primes` of limb j of the extended basis at `level`
  int prime_index(int level, int j) const { return j < level ? j : L + (j - level); }
  int key_limb(int level, int j) const { return j < level ? j : key_level(level) + (j - level); }
};

int nthreads(int t) { return t > 0 ? t : omp_get_max_threads(); }

}  // namespace

extern "C" {

// Parameter set: N = 2^log2n (4..17), L ciphertext primes, dnum digits at the
// top level, K special primes, digit partition 0 or 1, ChaCha rounds (even).
// Returns a handle, or null for bad arguments or too few primes.
void* o2_create(int log2n, int L, int dnum, int K, int partition, int rounds) {
  if (log2n < 4 || log2n > 17 || L < 1 || K < 1 || dnum < 1 || dnum > L || partition < 0 || partition > 1 ||
      rounds < 0 || (rounds & 1))
    return nullptr;
  Ctx* c = new Ctx;
  c->logn = log2n;
  c->N = 1u << log2n;
  c->L = L;
  c->dnum = dnum;
  c->K = K;
  c->partition = partition;
  c->rounds = rounds;
  c->primes = prime_chain(c->N, L + K);
  if ((int)c->primes.size() != L + K) {
    delete c;
    return nullptr;
  }
  c->ntt.resize(L + K);
#pragma omp parallel for schedule(dynamic)
  for (int k = 0; k < L + K; ++k) c->ntt[k].init(c->primes[k], c->N, log2n);
  return c;
}

void o2_destroy(void* h) { delete static_cast<Ctx*>(h); }

// primes[L+K] and psi[L+K] of the parameter set.
void o2_tables(void* h, uint32_t* primes, uint32_t* psi) {
  const Ctx* c = static_cast<Ctx*>(h);
  for (int k = 0; k < c->L + c->K; ++k) {
    primes[k] = c->primes[k];
    psi[k] = c->ntt[k].psi;
  }
}

// In-place forward (inverse = 0) or inverse NTT of N words mod prime `k`
// (0..L+K-1). Returns 0, or -1 for a bad index.
int o2_ntt(void* h, int k, uint32_t* x, int inverse) {
  const Ctx* c = static_cast<Ctx*>(h);
  if (k < 0 || k >= c->L + c->K) return -1;
  if (inverse)
    c->ntt[k].inverse(x);
  else
    c->ntt[k].forward(x);
  return 0;
}

// `nblocks` consecutive ChaCha blocks from `counter` for a 32-byte key (eight
// little-endian words) and a 3-word nonce: out[nblocks][16].
void o2_chacha_blocks(const uint8_t* key, uint32_t counter, const uint32_t* nonce, int rounds, int nblocks,
                      uint32_t* out) {
  u32 kw[8];
  for (int w = 0; w < 8; ++w)
    kw[w] = (u32)key[4 * w] | ((u32)key[4 * w + 1] << 8) | ((u32)key[4 * w + 2] << 16) | ((u32)key[4 * w + 3] << 24);
  for (int b = 0; b < nblocks; ++b) chacha_block(kw, counter + (u32)b, nonce, rounds, out + 16 * b);
}

// One key switch of ct [2][level][N] (evaluation form, canonical residues:
// word i of limb j below that limb's prime; the key's words likewise)
// under the key of odd Galois element `galois` (< 2N; 1 = relinearisation
// shape). evk_b: [beta_key][key_level+K][N], beta_key the key's digit count;
// the a half is evk_a (same shape) or, when evk_a is null, regenerated from
// the 32-byte `seed`. out: [2][level][N]. `threads` OpenMP threads (0: the
// runtime's default). Returns 0, or -1 for bad arguments.
int o2_keyswitch(void* h, int level, const uint32_t* ct, uint32_t galois, const uint32_t* evk_b,
                 const uint32_t* evk_a, const uint8_t* seed, uint32_t* out, int threads) {
  const Ctx* c = static_cast<Ctx*>(h);
  if (c == nullptr || level < 1 || level > c->L || (galois & 1u) == 0 || galois >= 2 * c->N) return -1;
  if (evk_a == nullptr && seed == nullptr) return -1;
  const int nt = nthreads(threads);
  const u32 N = c->N, mask = N - 1, half = (galois - 1) / 2;
  const size_t NN = N;
  const int K = c->K, lk = level + K, a = c->alpha(level), klk = c->key_level(level) + K;
  const int beta = (level + a - 1) / a;
  const u32* c0 = ct;
  const u32* c1 = ct + (size_t)level * NN;
  auto modulus = [&](int j) { return c->primes[c->prime_index(level, j)]; };
  auto src = [&](u32 n) { return (n * galois + half) & mask; };  // X -> X^k; N divides 2^32

  // 1. c1 to coefficients
  std::vector<u32> coef((size_t)level * NN);
#pragma omp parallel for schedule(dynamic) num_threads(nt)
  for (int i = 0; i < level; ++i) {
    std::memcpy(&coef[i * NN], c1 + i * NN, NN * 4);
    c->ntt[i].inverse(&coef[i * NN]);
  }

  // 2. ModUp: y_i = [coef_i (Q_d/q_i)^-1]_{q_i} for i in digit d, then
  // ext[d][t] = NTT((sum_i y_i [Q_d/q_i]_t) mod t) for every other modulus t;
  // the digit's own limbs are c1's limbs as given.
#pragma omp parallel for schedule(dynamic) num_threads(nt)
  for (int i = 0; i < level; ++i) {
    const int d = i / a, i0 = d * a, i1 = (i0 + a < level) ? i0 + a : level;
    const u32 qi = c->primes[i];
    u32 qhat = 1;
    for (int k = i0; k < i1; ++k)
      if (k != i) qhat = mulm(qhat, c->primes[k] % qi, qi);
    const u32 s = invm(qhat, qi);
    for (u32 n = 0; n < N; ++n) coef[i * NN + n] = mulm(coef[i * NN + n], s, qi);
  }
  std::vector<u32> ext((size_t)beta * lk * NN);
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt)
  for (int d = 0; d < beta; ++d) {
    for (int j = 0; j < lk; ++j) {
      const int i0 = d * a, i1 = (i0 + a < level) ? i0 + a : level;
      u32* dst = &ext[((size_t)d * lk + j) * NN];
      if (j >= i0 && j < i1) {
        std::memcpy(dst, c1 + j * NN, NN * 4);
        continue;
      }
      const u32 t = modulus(j);
      std::vector<u32> qhat_t(i1 - i0);
      for (int i = i0; i < i1; ++i) {
        u32 v = 1;
        for (int k = i0; k < i1; ++k)
          if (k != i) v = mulm(v, c->primes[k] % t, t);
        qhat_t[i - i0] = v;
      }
      for (u32 n = 0; n < N; ++n) {
        u32 z = 0;
        for (int i = i0; i < i1; ++i) z = addm(z, mulm(coef[i * NN + n], qhat_t[i - i0], t), t);
        dst[n] = z;
      }
      c->ntt[c->prime_index(level, j)].forward(dst);
    }
  }

  // 3-4. automorphism of ext and the inner product with (b_d, a_d)
  u32 seed_words[8] = {0};
  if (seed != nullptr)
    for (int w = 0; w < 8; ++w)
      seed_words[w] = (u32)seed[4 * w] | ((u32)seed[4 * w + 1] << 8) | ((u32)seed[4 * w + 2] << 16) |
                      ((u32)seed[4 * w + 3] << 24);
  std::vector<u32> acc((size_t)2 * lk * NN, 0);
#pragma omp parallel for schedule(dynamic) num_threads(nt)
  for (int j = 0; j < lk; ++j) {
    const u32 r = modulus(j);
    const int kj = c->key_limb(level, j);
    std::vector<u32> key_a(NN);
    u32* acc0 = &acc[(size_t)j * NN];
    u32* acc1 = &acc[((size_t)lk + j) * NN];
    for (int d = 0; d < beta; ++d) {
      const u32* b = evk_b + ((size_t)d * klk + kj) * NN;
      if (evk_a != nullptr) {
        std::memcpy(key_a.data(), evk_a + ((size_t)d * klk + kj) * NN, NN * 4);
      } else {
        const u32 nonce[3] = {0u, (u32)d, (u32)kj};
        for (u32 blk = 0; blk < N / 8; ++blk) {
          u32 w[16];
          chacha_block(seed_words, blk, nonce, c->rounds, w);
          for (int k = 0; k < 8; ++k) key_a[8 * blk + k] = (u32)((((u64)w[2 * k + 1] << 32) | w[2 * k]) % r);
        }
      }
      const u32* e = &ext[((size_t)d * lk + j) * NN];
      for (u32 n = 0; n < N; ++n) {
        const u32 x = e[src(n)];
        acc0[n] = addm(acc0[n], mulm(x, b[n], r), r);
        acc1[n] = addm(acc1[n], mulm(x, key_a[n], r), r);
      }
    }
  }

  // 5. ModDown of both accumulators: y_t = [iNTT(acc on p_t) (P/p_t)^-1]_{p_t},
  // z_i = (sum_t y_t [P/p_t]_{q_i}) mod q_i, out[i] = (acc_i - NTT(z_i)) P^-1;
  // 6. out0 += the automorphism of c0.
  std::vector<u32> yp((size_t)2 * K * NN);
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt)
  for (int u = 0; u < 2; ++u) {
    for (int t = 0; t < K; ++t) {
      const u32 pt = c->primes[c->L + t];
      u32* x = &yp[((size_t)u * K + t) * NN];
      std::memcpy(x, &acc[((size_t)u * lk + level + t) * NN], NN * 4);
      c->ntt[c->L + t].inverse(x);
      u32 phat = 1;
      for (int k = 0; k < K; ++k)
        if (k != t) phat = mulm(phat, c->primes[c->L + k] % pt, pt);
      const u32 s = invm(phat, pt);
      for (u32 n = 0; n < N; ++n) x[n] = mulm(x[n], s, pt);
    }
  }
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt)
  for (int u = 0; u < 2; ++u) {
    for (int i = 0; i < level; ++i) {
      const u32 qi = c->primes[i];
      std::vector<u32> z(NN, 0);
      u32 p_mod_qi = 1;
      for (int t = 0; t < K; ++t) {
        u32 phat = 1;
        for (int k = 0; k < K; ++k)
          if (k != t) phat = mulm(phat, c->primes[c->L + k] % qi, qi);
        const u32* y = &yp[((size_t)u * K + t) * NN];
        for (u32 n = 0; n < N; ++n) z[n] = addm(z[n], mulm(y[n], phat, qi), qi);
        p_mod_qi = mulm(p_mod_qi, c->primes[c->L + t] % qi, qi);
      }
      c->ntt[i].forward(z.data());
      const u32 p_inv = invm(p_mod_qi, qi);
      const u32* ai = &acc[((size_t)u * lk + i) * NN];
      u32* o = out + ((size_t)u * level + i) * NN;
      for (u32 n = 0; n < N; ++n) {
        u32 v = mulm(subm(ai[n], z[n], qi), p_inv, qi);
        if (u == 0) v = addm(v, c0[(size_t)i * NN + src(n)], qi);
        o[n] = v;
      }
    }
  }
  return 0;
}

}  // extern "C"
