// C-ABI entry points and host-side construction of the constant tables.
//
// The tables follow the readings stated in include/pc.h: the descending
// prime rule for the 32-bit chain (Perseus README, opening paragraph: 32-bit
// kernels), psi = the smallest primitive 2N-th root, natural-order evaluation,
// digits of alpha(l) = ceil(l/dnum) primes, ModDown in floor form.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "internal.h"

// Workspace of pc_keyswitch_static, the entry point that allocates nothing: a
// file-scope device array. Every GPU the library runs on holds its own copy
// until the process ends. In host code the name `scratch` is only a stand-in:
// kernels get the address hipGetSymbolAddress returns for the current device.
static constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace pc {
namespace {

uint32_t mulmod(uint32_t a, uint32_t b, uint32_t r) { return (uint32_t)((uint64_t)a * b % r); }

uint32_t powmod(uint32_t a, uint64_t e, uint32_t r) {
  uint64_t x = 1, b = a % r;
  while (e) {
    if (e & 1) x = x * b % r;
    b = b * b % r;
    e >>= 1;
  }
  return (uint32_t)x;
}

uint32_t invmod(uint32_t a, uint32_t r) { return powmod(a, r - 2, r); }  // r prime

uint32_t shoup(uint32_t w, uint32_t r) { return (uint32_t)(((uint64_t)w << 32) / r); }

// Deterministic Miller-Rabin for n < 2^32 (bases 2, 7, 61).
bool is_prime32(uint32_t n) {
  if (n < 2) return false;
  for (uint32_t p : {2u, 3u, 5u, 7u, 11u, 13u, 61u})
    if (n % p == 0) return n == p;
  uint32_t d = n - 1;
  int s = 0;
  while ((d & 1) == 0) {
    d >>= 1;
    ++s;
  }
  for (uint32_t a : {2u, 7u, 61u}) {
    uint32_t x = powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool composite = true;
    for (int i = 1; i < s; ++i) {
      x = mulmod(x, x, n);
      if (x == n - 1) {
        composite = false;
        break;
      }
    }
    if (composite) return false;
  }
  return true;
}

// Smallest primitive 2N-th root of unity mod r: find one root r0, then take the
// minimum over its odd powers (exactly the primitive 2N-th roots).
uint32_t smallest_psi(uint32_t r, uint32_t N) {
  uint32_t r0 = 0;
  for (uint32_t g = 2; g < r; ++g) {
    r0 = powmod(g, (r - 1) / (2 * (uint64_t)N), r);
    if (powmod(r0, N, r) == r - 1) break;
  }
  const uint32_t r0sq = mulmod(r0, r0, r);
  uint32_t best = r0, x = r0;
  for (uint32_t t = 1; t < N; ++t) {
    x = mulmod(x, r0sq, r);
    best = std::min(best, x);
  }
  return best;
}

uint32_t neg_inv32(uint32_t r) {
  uint32_t x = 1;
  for (int i = 0; i < 5; ++i) x *= 2u - r * x;  // Newton: x = r^-1 mod 2^32
  return 0u - x;
}

uint32_t bitrev_host(uint32_t x, int bits) {
  uint32_t y = 0;
  for (int b = 0; b < bits; ++b) y |= ((x >> b) & 1u) << (bits - 1 - b);
  return y;
}

// product of primes q_i, i in [i0, i1) \ {skip}, modulo r
uint32_t prod_mod(const pc_params* p, int i0, int i1, int skip, uint32_t r) {
  uint32_t x = 1 % r;
  for (int i = i0; i < i1; ++i)
    if (i != skip) x = mulmod(x, p->primes[i] % r, r);
  return x;
}

uint32_t pow2_32(uint32_t r) { return (uint32_t)((uint64_t(1) << 32) % r); }

int build_tables(pc_params* p) {
  const uint32_t N = p->N, L = p->L, K = p->K, P = L + K;
  const int n = (int)p->log2n;
  p->psi.resize(P);
  p->h_rinv.resize(P);
  p->h_ninv.resize(P);
  p->h_ninvp.resize(P);
  p->h_r2.resize(P);
  p->h_tw_fwd.resize((size_t)P * N);
  p->h_tw_inv.resize((size_t)P * N);
  p->h_twm_fwd.resize((size_t)P * N);
  p->h_twm_inv.resize((size_t)P * N);
  p->h_twm_fblk.assign((size_t)P * N, 0);
  p->h_twm_iblk.assign((size_t)P * N, 0);
  for (uint32_t k = 0; k < P; ++k) {
    const uint32_t r = p->primes[k];
    const uint32_t psi = smallest_psi(r, N);
    const uint32_t psi_inv = invmod(psi, r);
    p->psi[k] = psi;
    p->h_rinv[k] = neg_inv32(r);
    p->h_ninv[k] = invmod(N % r, r);
    p->h_ninvp[k] = shoup(p->h_ninv[k], r);
    p->h_r2[k] = mulmod(pow2_32(r), pow2_32(r), r);
    // psi^e for e = 0..N-1, then scatter by bit reversal
    std::vector<uint32_t> pw(N), pwi(N);
    pw[0] = pwi[0] = 1;
    for (uint32_t e = 1; e < N; ++e) {
      pw[e] = mulmod(pw[e - 1], psi, r);
      pwi[e] = mulmod(pwi[e - 1], psi_inv, r);
    }
    uint32_t* tf = &p->h_tw_fwd[(size_t)k * N];
    uint32_t* ti = &p->h_tw_inv[(size_t)k * N];
    uint32_t* tfm = &p->h_twm_fwd[(size_t)k * N];
    uint32_t* tim = &p->h_twm_inv[(size_t)k * N];
    const uint32_t mont = pow2_32(r);
    for (uint32_t i = 0; i < N; ++i) {
      const uint32_t e = bitrev_host(i, n);
      tf[i] = pw[e];
      ti[i] = pwi[e];
      tfm[i] = mulmod(pw[e], mont, r);
      tim[i] = mulmod(pwi[e], mont, r);
    }
    // block-major copies: forward stage s, group g of block B -> entry
    // 2^(lrc+s) + B 2^s + g; inverse stage u, group g -> 2^(n-u-1) + B 2^(lrb-u-1) + g
    int lrc = 0, lrb = 0;
    pass_split(p->log2n, &lrc, &lrb);
    uint32_t* bf = &p->h_twm_fblk[(size_t)k * N];
    uint32_t* bi = &p->h_twm_iblk[(size_t)k * N];
    for (uint32_t B = 0; B < (1u << lrc); ++B) {
      const size_t base = (size_t)B << lrb;
      for (int st = 0; st < lrb; ++st) {
        for (uint32_t g = 0; g < (1u << st); ++g)
          bf[base + (1u << st) + g] = tfm[((size_t)1 << (lrc + st)) + ((size_t)B << st) + g];
        const int w = lrb - st - 1;  // inverse stage u = st has 2^(lrb-u-1) groups
        for (uint32_t g = 0; g < (1u << w); ++g)
          bi[base + (1u << w) + g] = tim[((size_t)1 << (n - st - 1)) + ((size_t)B << w) + g];
      }
    }
  }
  // ModUp tables per level
  p->mu_scale_off.assign(L + 1, 0);
  p->mu_bconv_off.assign(L + 1, 0);
  size_t so = 0, bo = 0;
  for (uint32_t l = 1; l <= L; ++l) {
    p->mu_scale_off[l] = so;
    p->mu_bconv_off[l] = bo;
    so += l;
    bo += (size_t)l * (l + K);
  }
  p->h_mu_scale.assign(so, 0);
  p->h_mu_scalep.assign(so, 0);
  p->h_mu_bconv.assign(bo, 0);
  p->h_mu_bconvw.assign(bo, 0);
  for (uint32_t l = 1; l <= L; ++l) {
    const int a = alpha_of(p, l);
    const uint32_t lk = l + K;
    for (uint32_t i = 0; i < l; ++i) {
      const int d = (int)i / a;
      const int i0 = d * a, i1 = std::min<int>(i0 + a, (int)l);
      const uint32_t qi = p->primes[i];
      const uint32_t qhat_inv = invmod(prod_mod(p, i0, i1, (int)i, qi), qi);
      const uint32_t sc = mulmod(p->h_ninv[i], qhat_inv, qi);
      p->h_mu_scale[p->mu_scale_off[l] + i] = sc;
      p->h_mu_scalep[p->mu_scale_off[l] + i] = shoup(sc, qi);
      for (uint32_t j = 0; j < lk; ++j) {
        if ((int)j >= i0 && (int)j < i1) continue;
        const uint32_t rj = j < l ? p->primes[j] : p->primes[L + (j - l)];
        const uint32_t qhat = prod_mod(p, i0, i1, (int)i, rj);
        const uint32_t pj = j < l ? j : L + (j - l);
        const size_t at = p->mu_bconv_off[l] + (size_t)i * lk + j;
        p->h_mu_bconv[at] = mulmod(qhat, pow2_32(rj), rj);
        p->h_mu_bconvw[at] = mulmod(p->h_mu_bconv[at], p->h_tw_fwd[(size_t)pj * N + 1], rj);
      }
    }
  }
  // ModDown tables: variant 0 (plain input), variant 1 (input carrying 2^-64)
  p->h_md_scale.assign(2 * K, 0);
  p->h_md_scalep.assign(2 * K, 0);
  p->h_md_bconv.assign((size_t)2 * K * L, 0);
  p->h_md_bconvw.assign((size_t)2 * K * L, 0);
  p->h_md_pinv.assign(2 * L, 0);
  p->h_md_pinvp.assign(2 * L, 0);
  for (int v = 0; v < 2; ++v) {
    for (uint32_t t = 0; t < K; ++t) {
      const uint32_t pt = p->primes[L + t];
      uint32_t phat = 1;
      for (uint32_t u = 0; u < K; ++u)
        if (u != t) phat = mulmod(phat, p->primes[L + u] % pt, pt);
      uint32_t sc = mulmod(p->h_ninv[L + t], invmod(phat, pt), pt);
      if (v == 1) sc = mulmod(sc, p->h_r2[L + t], pt);  // times 2^64
      p->h_md_scale[v * K + t] = sc;
      p->h_md_scalep[v * K + t] = shoup(sc, pt);
      for (uint32_t i = 0; i < L; ++i) {
        const uint32_t qi = p->primes[i];
        uint32_t ph = 1;
        for (uint32_t u = 0; u < K; ++u)
          if (u != t) ph = mulmod(ph, p->primes[L + u] % qi, qi);
        // (P/p_t) 2^32 S^-1 with S = 1 or 2^64, i.e. times 2^32 or 2^-32
        const uint32_t f = v == 0 ? pow2_32(qi) : invmod(pow2_32(qi), qi);
        const size_t at = ((size_t)v * K + t) * L + i;
        p->h_md_bconv[at] = mulmod(ph, f, qi);
        p->h_md_bconvw[at] = mulmod(p->h_md_bconv[at], p->h_tw_fwd[(size_t)i * N + 1], qi);
      }
    }
    for (uint32_t i = 0; i < L; ++i) {
      const uint32_t qi = p->primes[i];
      uint32_t Pm = 1;
      for (uint32_t u = 0; u < K; ++u) Pm = mulmod(Pm, p->primes[L + u] % qi, qi);
      uint32_t pinv = invmod(Pm, qi);
      if (v == 1) pinv = mulmod(pinv, p->h_r2[i], qi);
      p->h_md_pinv[v * L + i] = pinv;
      p->h_md_pinvp[v * L + i] = shoup(pinv, qi);
    }
  }
  // rescale tables: row l' = level - 1 (1 <= l' < L), entry i < l'
  p->h_rs_qlmod.assign((size_t)L * L, 0);
  p->h_rs_inv.assign((size_t)L * L, 0);
  p->h_rs_invp.assign((size_t)L * L, 0);
  for (uint32_t lp = 1; lp < L; ++lp) {
    const uint32_t ql = p->primes[lp];
    for (uint32_t i = 0; i < lp; ++i) {
      const uint32_t qi = p->primes[i], m = ql % qi, inv = invmod(m, qi);
      p->h_rs_qlmod[(size_t)lp * L + i] = m;
      p->h_rs_inv[(size_t)lp * L + i] = inv;
      p->h_rs_invp[(size_t)lp * L + i] = shoup(inv, qi);
    }
  }
  return PC_OK;
}

template <class T>
size_t append(std::vector<uint8_t>& blob, const std::vector<T>& v) {
  size_t off = (blob.size() + 255) & ~size_t(255);
  blob.resize(off + v.size() * sizeof(T));
  if (!v.empty()) memcpy(blob.data() + off, v.data(), v.size() * sizeof(T));
  return off;
}

int upload_tables(pc_params* p) {
  std::vector<uint32_t> r32(p->primes.begin(), p->primes.end());
  std::vector<uint8_t> blob;
  const size_t o_r = append(blob, r32), o_rinv = append(blob, p->h_rinv), o_ninv = append(blob, p->h_ninv),
               o_ninvp = append(blob, p->h_ninvp), o_r2 = append(blob, p->h_r2);
  const size_t o_tf = append(blob, p->h_twm_fwd), o_ti = append(blob, p->h_twm_inv);
  const size_t o_bf = append(blob, p->h_twm_fblk), o_bi = append(blob, p->h_twm_iblk);
  const size_t o_ms = append(blob, p->h_mu_scale), o_msp = append(blob, p->h_mu_scalep),
               o_mb = append(blob, p->h_mu_bconv);
  const size_t o_ds = append(blob, p->h_md_scale), o_dsp = append(blob, p->h_md_scalep),
               o_db = append(blob, p->h_md_bconv), o_dp = append(blob, p->h_md_pinv),
               o_dpp = append(blob, p->h_md_pinvp);
  const size_t o_mbw = append(blob, p->h_mu_bconvw), o_dbw = append(blob, p->h_md_bconvw);
  void* d = nullptr;
  if (hipMalloc(&d, blob.size()) != hipSuccess) return PC_ENOMEM;
  if (hipMemcpy(d, blob.data(), blob.size(), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(d);
    return PC_EDEVICE;
  }
  p->d_tables = d;
  auto at = [d](size_t off) { return reinterpret_cast<const uint32_t*>(static_cast<uint8_t*>(d) + off); };
  p->tabs = DevTables{at(o_r), at(o_rinv), at(o_ninv), at(o_ninvp), at(o_r2),
                      at(o_tf), at(o_ti),   at(o_bf),   at(o_bi)};
  p->ltabs = DevLevelTables{at(o_ms), at(o_msp), at(o_mb),  at(o_ds),  at(o_dsp),
                            at(o_db), at(o_dp),  at(o_dpp), at(o_mbw), at(o_dbw)};
  return PC_OK;
}

struct DeviceGuard {
  int old = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&old) != hipSuccess) {
      ok = false;
      return;
    }
    if (old != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (old >= 0 && hipGetDevice(&cur) == hipSuccess && cur != old) (void)hipSetDevice(old);
  }
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current (at params creation, or on the first static call).
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices] = {};

int scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxScratchDevices) return PC_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return PC_EDEVICE;
    }
    g_scratch[device] = ptr;
  }
  *out = g_scratch[device];
  return PC_OK;
}

// Device buffers are moved in 16-byte vectors: every device pointer of the ABI
// must be 16-byte aligned.
bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15u) != 0; }

}  // namespace

size_t ks_workspace_bytes(const pc_params* p, uint32_t level, uint32_t batch, uint32_t items) {
  const size_t N = p->N, l = level, K = p->K, lk = l + K, beta = (size_t)beta_of(p, level);
  size_t b = 0;
  b += align256(batch * l * (N + kLimbPad) * 4);
  b += 2 * align256(batch * beta * lk * N * 4);
  b += align256(items * 2 * lk * N * 4);
  b += align256(items * 2 * K * (N + kLimbPad) * 4);
  b += align256(items * 2 * l * N * 4);
  return b;
}

KsWorkspace ks_workspace_carve(const pc_params* p, void* base, uint32_t level, uint32_t batch, uint32_t items) {
  const size_t N = p->N, l = level, K = p->K, lk = l + K, beta = (size_t)beta_of(p, level);
  uint8_t* c = static_cast<uint8_t*>(base);
  KsWorkspace w;
  auto take = [&c](size_t bytes) {
    uint32_t* r = reinterpret_cast<uint32_t*>(c);
    c += align256(bytes);
    return r;
  };
  w.y = take(batch * l * (N + kLimbPad) * 4);
  w.tmp = take(batch * beta * lk * N * 4);
  w.ext = take(batch * beta * lk * N * 4);
  w.acc = take(items * 2 * lk * N * 4);
  w.y2 = take(items * 2 * K * (N + kLimbPad) * 4);
  w.tmp2 = take(items * 2 * l * N * 4);
  return w;
}

// Workspace of a homomorphic multiplication of `batch` pairs at level l: the
// tensor [batch][3][l][N] (d0, d2, d1), a [batch][2][l][N] buffer R for the
// relinearised pair's last limbs and then the rescale's column-pass output
// [2 batch][l-1][N], then the key switch's own workspace (whose ModUp buffer y,
// free after ModUp, takes the rescale's dropped limbs [2 batch][N]).
size_t hm_workspace_bytes(const pc_params* p, uint32_t level, uint32_t batch) {
  const size_t N = p->N, l = level;
  return align256(batch * 3 * l * N * 4) + align256(batch * 2 * l * N * 4) + ks_workspace_bytes(p, level, batch, batch);
}

// Workspace of a linear transform with n1 baby and n2 giant steps at level l:
// the key-switch workspace of the baby steps (one ciphertext, n1 - 1 keys; its
// ModDown buffers also serve the final ModDown), inner [2][n2][l+K][N], the
// giant-step sum [2][l+K][N], and for n2 > 1 the ModDown outputs
// [n2-1][l][N] and the key-switch workspace of the giant steps.
size_t lt_workspace_bytes(const pc_params* p, uint32_t level, uint32_t n1, uint32_t n2) {
  const size_t N = p->N, lk = level + p->K;
  size_t b = ks_workspace_bytes(p, level, 1, std::max<uint32_t>(1, n1 - 1));
  b += align256(2 * n2 * lk * N * 4) + align256(2 * lk * N * 4);
  if (n2 > 1) b += align256((n2 - 1) * (size_t)level * N * 4) + ks_workspace_bytes(p, level, n2 - 1, n2 - 1);
  return b;
}

const char* const kKernelNames[KID_COUNT] = {
    "ntt_fwd_col",     "ntt_fwd_blk",     "ntt_inv_blk",     "ntt_inv_col",    "modup_inv_blk",
    "modup_inv_col",   "modup_bconv",     "modup_fwd_blk",   "inner_product",  "moddown_inv_blk",
    "moddown_inv_col", "moddown_bconv",   "moddown_fwd_blk", "chacha_expand",  "keygen",
    "tensor",          "rescale_gather",  "rescale_col",     "rescale_blk",    "bsgs_baby",
    "bsgs_giant",      "seg_copy",        "moddown_rescale", "expand_key",     "modup_ip"};

static hipEvent_t prof_event(const pc_params* p) {
  if (p->prof_used == p->prof_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    p->prof_pool.push_back(e);
  }
  return p->prof_pool[p->prof_used++];
}

LaunchTimer::LaunchTimer(const pc_params* params, int kid, hipStream_t stream) : p(params), kernel(kid), s(stream) {
  if (p->prof_on) {
    start = prof_event(p);
    if (start) (void)hipEventRecord(start, s);
  }
}

LaunchTimer::~LaunchTimer() {
  if (p->prof_on && start) {
    hipEvent_t stop = prof_event(p);
    if (stop && hipEventRecord(stop, s) == hipSuccess) p->prof_recs.push_back({kernel, start, stop});
  }
}

// ModUp, inner product and ModDown of `batch` ciphertexts (c0 of ciphertext z
// at ct + z ct_stride, c1 at + c1_off) under `nkeys` keys; out is
// [nkeys][batch][2][l][N] and the workspace at `base` is carved for
// (level, batch, nkeys * batch).
hipError_t launch_keyswitch(const pc_params* p, const uint32_t* ct, uint64_t ct_stride, uint32_t c1_off,
                            uint32_t batch, uint32_t level, const KeyRef* keys, uint32_t nkeys,
                            const uint32_t* galois, void* base, uint32_t* out, hipStream_t s) {
  KsWorkspace ws = ks_workspace_carve(p, base, level, batch, nkeys * batch);
  // segment layout for gathers of single ciphertexts (hoisted keys); a batch
  // spreads its stores over more lines than the gathers save (measured slower)
  for (uint32_t k = 0; k < nkeys; ++k) ws.seg = ws.seg || (batch == 1 && keys[k].galois != 1u);
  hipError_t e = launch_modup_ip(p, ct, ct_stride, c1_off, batch, level, ws, keys, nkeys, s);
  if (e != hipSuccess) return e;
  // with the segment layout (one ciphertext), the combine pass gathers c0 from
  // a segment-layout copy in y, which ModUp no longer needs
  if (ws.seg) {
    e = launch_seg_copy(p, ct, level, ws.y, s);
    if (e != hipSuccess) return e;
  }
  const size_t lk = level + p->K;
  for (uint32_t k0 = 0; k0 < nkeys; k0 += kMaxKeysPerLaunch) {
    const uint32_t nk = std::min<uint32_t>(kMaxKeysPerLaunch, nkeys - k0);
    const size_t item0 = (size_t)k0 * batch;
    e = launch_moddown(p, ws.acc + item0 * 2 * lk * p->N, nk * batch, 2, level, 1, out + item0 * 2 * level * p->N,
                       ws, ws.seg ? ws.y : ct, ct_stride, batch, galois + k0, s, ws.seg);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pc

using namespace pc;

extern "C" {

const char* pc_strerror(int code) {
  switch (code) {
    case PC_OK: return "ok";
    case PC_EINVAL: return "invalid argument";
    case PC_ENOMEM: return "out of memory";
    case PC_EDEVICE: return "device error (HIP call failed or no device)";
    case PC_EUNSUPPORTED: return "unsupported shape";
    default: return "unknown error";
  }
}

int pc_params_create(const pc_params_desc* desc, int device, pc_params** out) {
  if (desc == nullptr || out == nullptr) return PC_EINVAL;
  *out = nullptr;
  const uint32_t n = desc->log2n;
  if (n != 12 && n != 16 && n != 17) return PC_EUNSUPPORTED;
  if (desc->L < 1 || desc->K < 1 || desc->dnum < 1 || desc->dnum > desc->L) return PC_EINVAL;
  if (desc->dnum > (uint32_t)kMaxDigits) return PC_EUNSUPPORTED;
  if (desc->K > (uint32_t)kMaxSpecial) return PC_EUNSUPPORTED;
  if ((desc->L + desc->dnum - 1) / desc->dnum > (uint32_t)kMaxAlpha) return PC_EUNSUPPORTED;
  if (desc->L + desc->K > (uint32_t)kMaxLimbsPerLaunch - 1) return PC_EUNSUPPORTED;
  if (desc->partition > 1) return PC_EINVAL;
  const uint32_t rounds = desc->chacha_rounds ? desc->chacha_rounds : 12;
  if (rounds != 12 && rounds != 20) return PC_EUNSUPPORTED;
  const uint32_t max_hoist = desc->max_hoist ? desc->max_hoist : 1;
  if (max_hoist > (uint32_t)kMaxKeysPerLaunch) return PC_EUNSUPPORTED;
  pc_params* p = new (std::nothrow) pc_params();
  if (p == nullptr) return PC_ENOMEM;
  p->log2n = n;
  p->N = 1u << n;
  p->L = desc->L;
  p->K = desc->K;
  p->dnum = desc->dnum;
  p->max_batch = desc->max_batch ? desc->max_batch : 1;
  p->max_hoist = max_hoist;
  p->chacha_rounds = rounds;
  p->partition = desc->partition;
  const uint32_t count = p->L + p->K;
  const uint64_t m = 2ull * p->N;
  if (desc->primes != nullptr) {
    for (uint32_t k = 0; k < count; ++k) {
      const uint32_t r = desc->primes[k];
      if (r <= (1u << 30) || r >= (1u << 31) || r % m != 1 || !is_prime32(r)) {
        delete p;
        return PC_EINVAL;
      }
      for (uint32_t u = 0; u < k; ++u)
        if (desc->primes[u] == r) {
          delete p;
          return PC_EINVAL;
        }
      p->primes.push_back(r);
    }
  } else {
    uint64_t c = ((1ull << 31) - 2) / m * m + 1;
    while (p->primes.size() < count && c > (1u << 30)) {
      if (is_prime32((uint32_t)c)) p->primes.push_back((uint32_t)c);
      c -= m;
    }
    if (p->primes.size() < count) {
      delete p;
      return PC_EUNSUPPORTED;
    }
  }
  build_tables(p);
  {
    // the arena fits a key switch of max_batch x max_hoist and an HMult of
    // max_batch pairs at every level (with ceil(l/dnum) primes per digit a
    // lower level can have more digits, and so a larger ext, than the top),
    // and an NTT of every prime
    size_t need = (size_t)2 * count * p->N * 4;
    for (uint32_t l = 1; l <= p->L; ++l) {
      need = std::max(need, ks_workspace_bytes(p, l, p->max_batch, p->max_batch * p->max_hoist));
      if (l >= 2) need = std::max(need, hm_workspace_bytes(p, l, p->max_batch));
    }
    p->arena_bytes = need;
  }
  if (device >= 0) {
    DeviceGuard g(device);
    if (!g.ok) {
      delete p;
      return PC_EDEVICE;
    }
    p->device = device;
    int rc = upload_tables(p);
    if (rc != PC_OK) {
      delete p;
      return rc;
    }
    if (hipMalloc(&p->arena, p->arena_bytes) != hipSuccess) {
      (void)hipGetLastError();  // do not leave the failure for a later launch check to report
      (void)hipFree(p->d_tables);
      delete p;
      return PC_ENOMEM;
    }
    // the static entry point's scratch address on this device (a failure is
    // reported by that entry point, which retries the lookup)
    void* sp = nullptr;
    (void)scratch_address(device, &sp);
  }
  *out = p;
  return PC_OK;
}

void pc_params_destroy(pc_params* p) {
  if (p == nullptr) return;
  if (p->device >= 0) {
    DeviceGuard g(p->device);
    for (hipEvent_t e : p->prof_pool) (void)hipEventDestroy(e);
    if (p->arena) (void)hipFree(p->arena);
    if (p->d_tables) (void)hipFree(p->d_tables);
  }
  delete p;
}

int pc_profile_begin(const pc_params* p) {
  if (p == nullptr) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  p->prof_recs.clear();
  p->prof_used = 0;
  p->prof_on = true;
  return PC_OK;
}

int pc_profile_end(const pc_params* p, pc_kernel_stat* stats, uint32_t max_stats, uint32_t* count) {
  if (p == nullptr || count == nullptr || (stats == nullptr && max_stats > 0)) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  p->prof_on = false;
  double ms[KID_COUNT] = {0};
  uint32_t n[KID_COUNT] = {0};
  int rc = PC_OK;
  for (const auto& r : p->prof_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) {
      rc = PC_EDEVICE;
      continue;
    }
    ms[r.kernel] += t;
    n[r.kernel] += 1;
  }
  p->prof_recs.clear();
  p->prof_used = 0;
  uint32_t c = 0;
  for (int k = 0; k < KID_COUNT; ++k) {
    if (n[k] == 0) continue;
    if (c < max_stats) stats[c] = pc_kernel_stat{kKernelNames[k], n[k], ms[k]};
    ++c;
  }
  *count = c < max_stats ? c : max_stats;
  return rc;
}

int pc_params_get(const pc_params* p, int what, uint32_t arg, void* dst, size_t bytes) {
  if (p == nullptr || dst == nullptr) return PC_EINVAL;
  const uint32_t count = p->L + p->K;
  switch (what) {
    case PC_GET_N:
      if (bytes != 4) return PC_EINVAL;
      memcpy(dst, &p->N, 4);
      return PC_OK;
    case PC_GET_PRIMES:
      if (bytes != count * 4) return PC_EINVAL;
      memcpy(dst, p->primes.data(), bytes);
      return PC_OK;
    case PC_GET_PSI:
      if (bytes != count * 4) return PC_EINVAL;
      memcpy(dst, p->psi.data(), bytes);
      return PC_OK;
    case PC_GET_ALPHA:
    case PC_GET_BETA: {
      if (bytes != 4 || arg < 1 || arg > p->L) return PC_EINVAL;
      const uint32_t v = (uint32_t)(what == PC_GET_ALPHA ? alpha_of(p, arg) : beta_of(p, arg));
      memcpy(dst, &v, 4);
      return PC_OK;
    }
    case PC_GET_WORKSPACE_BYTES: {
      if (bytes != 8 || arg < 1 || arg > p->L) return PC_EINVAL;
      const uint64_t v = ks_workspace_bytes(p, arg, p->max_batch, p->max_batch * p->max_hoist);
      memcpy(dst, &v, 8);
      return PC_OK;
    }
    case PC_GET_ARENA_BYTES: {
      if (bytes != 8) return PC_EINVAL;
      const uint64_t v = p->arena_bytes;
      memcpy(dst, &v, 8);
      return PC_OK;
    }
    case PC_GET_LT_WORKSPACE_BYTES: {
      const uint32_t level = arg & 0xff, n1 = (arg >> 8) & 0xff, n2 = arg >> 16;
      if (bytes != 8 || level < 1 || level > p->L || n1 < 1 || n2 < 1) return PC_EINVAL;
      const uint64_t v = lt_workspace_bytes(p, level, n1, n2);
      memcpy(dst, &v, 8);
      return PC_OK;
    }
    case PC_GET_DEVICE_TABLE:
      if (arg >= count || bytes != (size_t)p->N * 4) return PC_EINVAL;
      memcpy(dst, &p->h_tw_fwd[(size_t)arg * p->N], bytes);
      return PC_OK;
    default:
      return PC_EINVAL;
  }
}

static int ntt_common(const pc_params* p, uint32_t* data, const uint32_t* prime_idx, uint32_t nlimbs, uint32_t count,
                      void* stream, bool inverse) {
  if (p == nullptr || data == nullptr || prime_idx == nullptr || misaligned(data)) return PC_EINVAL;
  for (uint32_t z = 0; z < nlimbs; ++z)
    if (prime_idx[z] >= p->L + p->K) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  const size_t total = (size_t)nlimbs * count;
  if (total == 0) return PC_OK;
  if (total > 0xffffffffull) return PC_EINVAL;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  // polynomial c, limb z uses prime_idx[z]; the arena holds the transform's scratch
  std::vector<uint32_t> idx(total);
  for (size_t k = 0; k < total; ++k) idx[k] = prime_idx[k % nlimbs];
  const uint32_t chunk = (uint32_t)std::min<size_t>(total, p->arena_bytes / ((size_t)p->N * 4));
  for (size_t base = 0; base < total; base += chunk) {
    const uint32_t cnt = (uint32_t)std::min<size_t>(chunk, total - base);
    if (launch_ntt(p, data + base * p->N, static_cast<uint32_t*>(p->arena), idx.data() + base, cnt, inverse,
                   (hipStream_t)stream) != hipSuccess)
      return PC_EDEVICE;
  }
  return PC_OK;
}

int pc_ntt(const pc_params* p, uint32_t* data, const uint32_t* prime_idx, uint32_t nlimbs, uint32_t count,
           void* stream) {
  return ntt_common(p, data, prime_idx, nlimbs, count, stream, false);
}

int pc_intt(const pc_params* p, uint32_t* data, const uint32_t* prime_idx, uint32_t nlimbs, uint32_t count,
            void* stream) {
  return ntt_common(p, data, prime_idx, nlimbs, count, stream, true);
}

int pc_modup(const pc_params* p, const uint32_t* c1, uint32_t level, uint32_t* ext, void* stream) {
  if (p == nullptr || c1 == nullptr || ext == nullptr || misaligned(c1) || misaligned(ext)) return PC_EINVAL;
  if (level < 1 || level > p->L) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  KsWorkspace ws = ks_workspace_carve(p, p->arena, level, 1, 1);
  ws.ext = ext;
  hipStream_t s = (hipStream_t)stream;
  if (launch_modup(p, c1, 0, 0, 1, level, ws, s) != hipSuccess) return PC_EDEVICE;
  const int a = alpha_of(p, level), beta = beta_of(p, level);
  const size_t lk = level + p->K, N = p->N;
  for (int d = 0; d < beta; ++d) {
    const int i0 = d * a, i1 = std::min<int>(i0 + a, (int)level);
    if (hipMemcpyAsync(ext + ((size_t)d * lk + i0) * N, c1 + (size_t)i0 * N, (size_t)(i1 - i0) * N * 4,
                       hipMemcpyDeviceToDevice, s) != hipSuccess)
      return PC_EDEVICE;
  }
  return PC_OK;
}

int pc_moddown(const pc_params* p, const uint32_t* acc, uint32_t level, uint32_t* out, void* stream) {
  if (p == nullptr || acc == nullptr || out == nullptr || misaligned(acc) || misaligned(out)) return PC_EINVAL;
  if (level < 1 || level > p->L) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  KsWorkspace ws = ks_workspace_carve(p, p->arena, level, 1, 1);
  if (launch_moddown(p, acc, 1, 1, level, 0, out, ws, nullptr, 0, 1, nullptr, (hipStream_t)stream) != hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

// Validates the arguments of a batched / hoisted key switch and fills keys[]
// (a->nkeys entries; nkeys <= max_hoist <= kMaxKeysPerLaunch). No allocation.
static int ks_args_keys(const pc_params* p, const pc_ks_args* a, KeyRef* keys) {
  if (p == nullptr || a == nullptr || a->ct == nullptr || a->out == nullptr || a->evk_b == nullptr ||
      a->galois == nullptr)
    return PC_EINVAL;
  if (misaligned(a->ct) || misaligned(a->out) || misaligned(a->workspace)) return PC_EINVAL;
  if (a->level < 1 || a->level > p->L) return PC_EINVAL;
  if (a->batch < 1 || a->batch > p->max_batch) return PC_EINVAL;
  if (a->nkeys < 1 || a->nkeys > p->max_hoist || a->nkeys > (uint32_t)kMaxKeysPerLaunch) return PC_EINVAL;
  if (a->evk_a == nullptr && a->seeds == nullptr) return PC_EINVAL;
  for (uint32_t k = 0; k < a->nkeys; ++k) {
    const uint32_t gk = a->galois[k];
    if ((gk & 1u) == 0 || gk >= 2 * p->N) return PC_EINVAL;
    if (a->evk_b[k] == nullptr || misaligned(a->evk_b[k])) return PC_EINVAL;
    keys[k].b = a->evk_b[k];
    keys[k].a = nullptr;
    if (a->evk_a != nullptr) {
      if (a->evk_a[k] == nullptr || misaligned(a->evk_a[k])) return PC_EINVAL;
      keys[k].a = a->evk_a[k];
    }
    if (a->seeds != nullptr) {
      for (int w = 0; w < 8; ++w) {
        const uint8_t* s = a->seeds + 32 * k + 4 * w;
        keys[k].seed[w] = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
      }
    } else {
      memset(keys[k].seed, 0, sizeof(keys[k].seed));
    }
    keys[k].galois = gk;
  }
  return PC_OK;
}

int pc_keyswitch_ex(const pc_params* p, const pc_ks_args* a, void* stream) {
  KeyRef keys[kMaxKeysPerLaunch];
  const int rc = ks_args_keys(p, a, keys);
  if (rc != PC_OK) return rc;
  if (p->device < 0) return PC_EDEVICE;
  const uint32_t items = a->nkeys * a->batch;
  const size_t need = ks_workspace_bytes(p, a->level, a->batch, items);
  void* base = p->arena;
  if (a->workspace != nullptr) {
    if (a->workspace_bytes < need) return PC_EINVAL;
    base = a->workspace;
  } else if (need > p->arena_bytes) {
    return PC_EINVAL;
  }
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  const uint64_t ct_stride = 2ull * a->level * p->N;
  if (launch_keyswitch(p, a->ct, ct_stride, a->level * p->N, a->batch, a->level, keys, a->nkeys, a->galois, base,
                       a->out, (hipStream_t)stream) != hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

int pc_keyswitch_static(const pc_params* p, const pc_ks_args* a, void* stream) {
  KeyRef keys[kMaxKeysPerLaunch];
  const int rc = ks_args_keys(p, a, keys);
  if (rc != PC_OK) return rc;
  if (a->workspace != nullptr || a->workspace_bytes != 0) return PC_EINVAL;  // the scratch is the workspace
  const size_t need = ks_workspace_bytes(p, a->level, a->batch, a->nkeys * a->batch);
  if (need > kScratchBytes) return PC_EUNSUPPORTED;
  if (p->device < 0) return PC_EDEVICE;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  void* base = nullptr;
  const int sr = scratch_address(p->device, &base);
  if (sr != PC_OK) return sr;
  const uint64_t ct_stride = 2ull * a->level * p->N;
  if (launch_keyswitch(p, a->ct, ct_stride, a->level * p->N, a->batch, a->level, keys, a->nkeys, a->galois, base,
                       a->out, (hipStream_t)stream) != hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

int pc_keyswitch(const pc_params* p, const uint32_t* ct, const uint32_t* evk_b, const uint8_t* evk_seed,
                 uint32_t level, uint32_t automorphism_idx, uint32_t* out, void* stream) {
  if (evk_seed == nullptr || evk_b == nullptr) return PC_EINVAL;
  const uint32_t* bl[1] = {evk_b};
  const uint32_t gl[1] = {automorphism_idx};
  pc_ks_args a;
  memset(&a, 0, sizeof(a));
  a.ct = ct;
  a.batch = 1;
  a.nkeys = 1;
  a.evk_b = bl;
  a.evk_a = nullptr;
  a.seeds = evk_seed;
  a.galois = gl;
  a.level = level;
  a.out = out;
  return pc_keyswitch_ex(p, &a, stream);
}

int pc_keygen(const pc_params* p, const uint8_t* seed, uint32_t level, uint32_t galois, const uint32_t* s_coef,
              const uint32_t* e_coef, uint32_t* evk_b, void* stream) {
  if (p == nullptr || seed == nullptr || s_coef == nullptr || e_coef == nullptr || evk_b == nullptr) return PC_EINVAL;
  if (misaligned(s_coef) || misaligned(e_coef) || misaligned(evk_b)) return PC_EINVAL;
  if (level < 1 || level > p->L) return PC_EINVAL;
  if ((galois & 1u) == 0 || galois >= 2 * p->N) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  const uint32_t lk = level + p->K, beta = (uint32_t)beta_of(p, level);
  const size_t N = p->N;
  // workspace: s [lk][N], e [beta][lk][N], NTT scratch [beta][lk][N]
  if ((size_t)(2 * beta + 1) * lk * N * 4 > p->arena_bytes) return PC_EINVAL;
  uint32_t* ws_s = static_cast<uint32_t*>(p->arena);
  uint32_t* ws_e = ws_s + (size_t)lk * N;
  uint32_t* ws_t = ws_e + (size_t)beta * lk * N;
  uint32_t key[8];
  for (int w = 0; w < 8; ++w)
    key[w] = (uint32_t)seed[4 * w] | ((uint32_t)seed[4 * w + 1] << 8) | ((uint32_t)seed[4 * w + 2] << 16) |
             ((uint32_t)seed[4 * w + 3] << 24);
  // prime index of every limb of the key basis, per digit block
  std::vector<uint32_t> pidx((size_t)beta * lk);
  for (uint32_t d = 0; d < beta; ++d)
    for (uint32_t j = 0; j < lk; ++j) pidx[(size_t)d * lk + j] = j < level ? j : p->L + (j - level);
  // [P]_{q_j} 2^32 mod q_j on the q-limbs (the gadget factor of the digit that owns q_j)
  std::vector<uint32_t> gm(lk, 0);
  for (uint32_t j = 0; j < level; ++j) {
    const uint32_t q = p->primes[j];
    gm[j] = mulmod(prod_mod(p, (int)p->L, (int)(p->L + p->K), -1, q), pow2_32(q), q);
  }
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(ws_s, s_coef, (size_t)lk * N * 4, hipMemcpyDeviceToDevice, s) != hipSuccess) return PC_EDEVICE;
  if (hipMemcpyAsync(ws_e, e_coef, (size_t)beta * lk * N * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return PC_EDEVICE;
  if (launch_ntt(p, ws_s, ws_t, pidx.data(), lk, false, s) != hipSuccess) return PC_EDEVICE;
  if (launch_ntt(p, ws_e, ws_t, pidx.data(), beta * lk, false, s) != hipSuccess) return PC_EDEVICE;
  if (launch_keygen(p, key, level, galois, ws_s, ws_e, gm.data(), evk_b, s) != hipSuccess) return PC_EDEVICE;
  return PC_OK;
}

int pc_tensor(const pc_params* p, const uint32_t* ct_a, const uint32_t* ct_b, uint32_t batch, uint32_t level,
              uint32_t* d, void* stream) {
  if (p == nullptr || ct_a == nullptr || ct_b == nullptr || d == nullptr) return PC_EINVAL;
  if (misaligned(ct_a) || misaligned(ct_b) || misaligned(d)) return PC_EINVAL;
  if (level < 1 || level > p->L || batch < 1 || batch > p->max_batch) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  const uint64_t ln = (uint64_t)level * p->N;
  const uint64_t off[3] = {0, ln, 2 * ln};
  if (launch_tensor(p, ct_a, 2 * ln, ct_b, 2 * ln, batch, level, d, 3 * ln, off, (hipStream_t)stream) != hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

int pc_rescale(const pc_params* p, const uint32_t* ct, uint32_t batch, uint32_t level, uint32_t* out, void* stream) {
  if (p == nullptr || ct == nullptr || out == nullptr || misaligned(ct) || misaligned(out)) return PC_EINVAL;
  if (level < 2 || level > p->L || batch < 1 || batch > p->max_batch) return PC_EINVAL;
  if (level - 1 > (uint32_t)kMaxRescaleLimbs || 2 * batch > (uint32_t)kMaxLimbsPerLaunch) return PC_EUNSUPPORTED;
  if (p->device < 0) return PC_EDEVICE;
  const size_t N = p->N;
  uint32_t* x = static_cast<uint32_t*>(p->arena);
  uint32_t* tmp = x + align256(2 * batch * N * 4) / 4;
  if (align256(2 * batch * N * 4) + (size_t)2 * batch * (level - 1) * N * 4 > p->arena_bytes) return PC_EINVAL;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  const uint64_t ln = (uint64_t)level * N;
  if (launch_rescale(p, ct, 2 * ln, (uint32_t)ln, nullptr, 0, batch, level, x, tmp, out, (hipStream_t)stream) !=
      hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

int pc_hmult(const pc_params* p, const uint32_t* ct_a, const uint32_t* ct_b, uint32_t batch, const uint32_t* evk_b,
             const uint8_t* evk_seed, uint32_t level, uint32_t* out, void* stream) {
  if (p == nullptr || ct_a == nullptr || ct_b == nullptr || evk_b == nullptr || evk_seed == nullptr || out == nullptr)
    return PC_EINVAL;
  if (misaligned(ct_a) || misaligned(ct_b) || misaligned(evk_b) || misaligned(out)) return PC_EINVAL;
  if (level < 2 || level > p->L || batch < 1 || batch > p->max_batch) return PC_EINVAL;
  if (level - 1 > (uint32_t)kMaxRescaleLimbs || 2 * batch > (uint32_t)kMaxLimbsPerLaunch) return PC_EUNSUPPORTED;
  if (p->device < 0) return PC_EDEVICE;
  if (hm_workspace_bytes(p, level, batch) > p->arena_bytes) return PC_EINVAL;
  KeyRef key;
  key.b = evk_b;
  key.a = nullptr;
  for (int w = 0; w < 8; ++w) {
    const uint8_t* sb = evk_seed + 4 * w;
    key.seed[w] = (uint32_t)sb[0] | ((uint32_t)sb[1] << 8) | ((uint32_t)sb[2] << 16) | ((uint32_t)sb[3] << 24);
  }
  key.galois = 1;
  const uint32_t one = 1;
  const size_t N = p->N, l = level;
  const uint64_t ln = (uint64_t)l * N;
  uint8_t* c = static_cast<uint8_t*>(p->arena);
  uint32_t* T = reinterpret_cast<uint32_t*>(c);  // [batch][3][l][N]: d0, d2, d1
  c += align256(batch * 3 * ln * 4);
  uint32_t* R = reinterpret_cast<uint32_t*>(c);  // [batch][2][l][N]: relinearised (d0, d2) without d1
  c += align256(batch * 2 * ln * 4);
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t off[3] = {0, 2 * ln, ln};
  if (launch_tensor(p, ct_a, 2 * ln, ct_b, 2 * ln, batch, level, T, 3 * ln, off, s) != hipSuccess) return PC_EDEVICE;
  // relinearisation of (d0, d2): ModUp and inner product as in a key switch;
  // ModDown brings down limb l-1 of both components first (into R), the
  // rescale turns it into the values to subtract (its column pass writes over
  // R, whose other limbs are never written), and one pass per limb < l-1
  // finishes ModDown and the rescale together
  const KsWorkspace ws = ks_workspace_carve(p, c, level, batch, batch);
  if (launch_modup_ip(p, T, 3 * ln, (uint32_t)ln, batch, level, ws, &key, 1, s) != hipSuccess) return PC_EDEVICE;
  if (launch_moddown(p, ws.acc, batch, 2, level, 1, R, ws, T, 3 * ln, batch, &one, s, false, level - 1) != hipSuccess)
    return PC_EDEVICE;
  if (launch_rescale(p, R, 2 * ln, (uint32_t)ln, T + 2 * ln, 3 * ln, batch, level, ws.y, R, out, s, false) !=
      hipSuccess)
    return PC_EDEVICE;
  if (launch_moddown_rescale(p, ws.acc, batch, level, ws, T, 3 * ln, T + 2 * ln, 3 * ln, R, out, s) != hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

static bool lt_keys(const pc_params* p, uint32_t n, const uint32_t* const* b, const uint8_t* seeds,
                    const uint32_t* galois, std::vector<KeyRef>& out) {
  out.resize(n);
  if (n == 0) return true;
  if (b == nullptr || seeds == nullptr || galois == nullptr) return false;
  for (uint32_t k = 0; k < n; ++k) {
    if (b[k] == nullptr || misaligned(b[k]) || (galois[k] & 1u) == 0 || galois[k] >= 2 * p->N) return false;
    out[k].b = b[k];
    out[k].a = nullptr;
    for (int w = 0; w < 8; ++w) {
      const uint8_t* sb = seeds + 32 * k + 4 * w;
      out[k].seed[w] = (uint32_t)sb[0] | ((uint32_t)sb[1] << 8) | ((uint32_t)sb[2] << 16) | ((uint32_t)sb[3] << 24);
    }
    out[k].galois = galois[k];
  }
  return true;
}

int pc_linear_transform(const pc_params* p, const pc_lt_args* a, void* stream) {
  if (p == nullptr || a == nullptr || a->ct == nullptr || a->diag == nullptr || a->out == nullptr) return PC_EINVAL;
  if (misaligned(a->ct) || misaligned(a->diag) || misaligned(a->out)) return PC_EINVAL;
  const uint32_t level = a->level, n1 = a->n1, n2 = a->n2;
  if (level < 1 || level > p->L || n1 < 1 || n1 > 8 || n2 < 1 || n2 > 32 || level + p->K > 64) return PC_EINVAL;
  std::vector<KeyRef> baby, giant;
  if (!lt_keys(p, n1 - 1, a->baby_b, a->baby_seeds, a->baby_galois, baby)) return PC_EINVAL;
  if (!lt_keys(p, n2 - 1, a->giant_b, a->giant_seeds, a->giant_galois, giant)) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  if (lt_workspace_bytes(p, level, n1, n2) > p->arena_bytes) return PC_EINVAL;
  const size_t N = p->N, l = level, lk = level + p->K;
  // per extended-basis limb: P 2^64 (q-limbs), 2^96 and 2^128 mod r
  std::vector<uint32_t> pm(lk, 0), m96(lk), m128(lk);
  for (uint32_t t = 0; t < lk; ++t) {
    const uint32_t r = t < level ? p->primes[t] : p->primes[p->L + t - level];
    if (t < level) pm[t] = mulmod(prod_mod(p, (int)p->L, (int)(p->L + p->K), -1, r), powmod(2, 64, r), r);
    m96[t] = powmod(2, 96, r);
    m128[t] = powmod(2, 128, r);
  }
  uint8_t* c = static_cast<uint8_t*>(p->arena);
  KsWorkspace ws1 = ks_workspace_carve(p, c, level, 1, std::max<uint32_t>(1, n1 - 1));
  for (const KeyRef& k : baby) ws1.seg = ws1.seg || k.galois != 1u;
  c += ks_workspace_bytes(p, level, 1, std::max<uint32_t>(1, n1 - 1));
  uint32_t* inner = reinterpret_cast<uint32_t*>(c);
  c += align256(2 * n2 * lk * N * 4);
  uint32_t* accqp = reinterpret_cast<uint32_t*>(c);
  c += align256(2 * lk * N * 4);
  uint32_t* d1 = reinterpret_cast<uint32_t*>(c);
  KsWorkspace ws2{};
  if (n2 > 1) {
    c += align256((n2 - 1) * l * N * 4);
    ws2 = ks_workspace_carve(p, c, level, n2 - 1, n2 - 1);
    for (const KeyRef& k : giant) ws2.seg = ws2.seg || k.galois != 1u;
  }
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t ln = (uint64_t)l * N;
  if (n1 > 1) {
    if (launch_modup(p, a->ct, 2 * ln, (uint32_t)ln, 1, level, ws1, s) != hipSuccess) return PC_EDEVICE;
    if (launch_inner_product(p, a->ct, 2 * ln, (uint32_t)ln, 1, level, ws1, baby.data(), n1 - 1, s) != hipSuccess)
      return PC_EDEVICE;
  }
  if (launch_bsgs_baby(p, a->ct, ws1.acc, a->diag, inner, level, n1, n2, a->baby_galois, pm.data(), m96.data(),
                       m128.data(), s) != hipSuccess)
    return PC_EDEVICE;
  if (n2 > 1) {
    // ModDown of inner_j,1 for j >= 1 (contiguous: inner is [u][j][l+K][N])
    if (launch_moddown(p, inner + (size_t)(n2 + 1) * lk * N, n2 - 1, 1, level, 0, d1, ws2, nullptr, 0, 1, nullptr, s) !=
        hipSuccess)
      return PC_EDEVICE;
    if (launch_modup(p, d1, ln, 0, n2 - 1, level, ws2, s) != hipSuccess) return PC_EDEVICE;
    // giant step j's key switches brought-down component j - 1: one launch, one ciphertext per key
    if (launch_inner_product(p, d1, ln, 0, 1, level, ws2, giant.data(), n2 - 1, s, true) != hipSuccess)
      return PC_EDEVICE;
  }
  if (launch_bsgs_giant(p, inner, n2 > 1 ? ws2.acc : nullptr, accqp, level, n2, a->giant_galois, pm.data(),
                        m96.data(), m128.data(), s) != hipSuccess)
    return PC_EDEVICE;
  if (launch_moddown(p, accqp, 1, 2, level, 0, a->out, ws1, nullptr, 0, 1, nullptr, s) != hipSuccess)
    return PC_EDEVICE;
  return PC_OK;
}

// ---------------------------------------------------------------------------
// key bundles
// ---------------------------------------------------------------------------

static void seed_words(const uint8_t* seed, uint32_t out[8]) {
  for (int w = 0; w < 8; ++w)
    out[w] = (uint32_t)seed[4 * w] | ((uint32_t)seed[4 * w + 1] << 8) | ((uint32_t)seed[4 * w + 2] << 16) |
             ((uint32_t)seed[4 * w + 3] << 24);
}

int pc_keyset_create(const pc_params* p, uint32_t level, uint32_t nkeys, const uint32_t* galois, uint32_t mode,
                     pc_keyset** out) {
  if (p == nullptr || galois == nullptr || out == nullptr) return PC_EINVAL;
  *out = nullptr;
  if (level < 1 || level > p->L || nkeys < 1 || nkeys > 256 || mode > PC_KEYSET_FULL) return PC_EINVAL;
  for (uint32_t k = 0; k < nkeys; ++k) {
    if ((galois[k] & 1u) == 0 || galois[k] >= 2 * p->N) return PC_EINVAL;
    for (uint32_t u = 0; u < k; ++u)
      if (galois[u] == galois[k]) return PC_EINVAL;
  }
  if (p->device < 0) return PC_EDEVICE;
  pc_keyset* ks = new (std::nothrow) pc_keyset();
  if (ks == nullptr) return PC_ENOMEM;
  ks->p = p;
  ks->key_level = key_level_of(p, level);
  ks->nkeys = nkeys;
  ks->mode = mode;
  ks->beta = (uint32_t)beta_of(p, ks->key_level);
  ks->lk = ks->key_level + p->K;
  ks->key_words = (size_t)ks->beta * ks->lk * p->N;
  ks->galois.assign(galois, galois + nkeys);
  ks->seeds.assign((size_t)nkeys * 32, 0);
  DeviceGuard g(p->device);
  if (!g.ok) {
    delete ks;
    return PC_EDEVICE;
  }
  const size_t bytes = (size_t)nkeys * (mode ? 2 : 1) * ks->key_words * 4;
  if (hipMalloc(&ks->mem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete ks;
    return PC_ENOMEM;
  }
  *out = ks;
  return PC_OK;
}

void pc_keyset_destroy(pc_keyset* ks) {
  if (ks == nullptr) return;
  if (ks->mem != nullptr) {
    DeviceGuard g(ks->p->device);
    (void)hipFree(ks->mem);
  }
  delete ks;
}

int pc_keyset_set(pc_keyset* ks, uint32_t idx, const uint32_t* evk_b, const uint8_t* seed, void* stream) {
  if (ks == nullptr || evk_b == nullptr || seed == nullptr || misaligned(evk_b) || idx >= ks->nkeys) return PC_EINVAL;
  const pc_params* p = ks->p;
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  memcpy(&ks->seeds[(size_t)idx * 32], seed, 32);
  if (hipMemcpyAsync(ks->b_of(idx), evk_b, ks->key_words * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return PC_EDEVICE;
  if (ks->mode == PC_KEYSET_FULL) {
    uint32_t key[8];
    seed_words(seed, key);
    if (launch_expand_key(p, key, ks->key_level, ks->a_of(idx), s) != hipSuccess) return PC_EDEVICE;
  }
  return PC_OK;
}

int pc_keyset_keygen(pc_keyset* ks, uint32_t idx, const uint8_t* seed, const uint32_t* s_coef, const uint32_t* e_coef,
                     void* stream) {
  if (ks == nullptr || seed == nullptr || idx >= ks->nkeys) return PC_EINVAL;
  const pc_params* p = ks->p;
  const int rc = pc_keygen(p, seed, ks->key_level, ks->galois[idx], s_coef, e_coef, ks->b_of(idx), stream);
  if (rc != PC_OK) return rc;
  memcpy(&ks->seeds[(size_t)idx * 32], seed, 32);
  if (ks->mode == PC_KEYSET_FULL) {
    DeviceGuard g(p->device);
    if (!g.ok) return PC_EDEVICE;
    uint32_t key[8];
    seed_words(seed, key);
    if (launch_expand_key(p, key, ks->key_level, ks->a_of(idx), (hipStream_t)stream) != hipSuccess)
      return PC_EDEVICE;
  }
  return PC_OK;
}

int pc_keyset_get(const pc_keyset* ks, int what, uint32_t arg, void* dst, size_t bytes) {
  if (ks == nullptr || dst == nullptr) return PC_EINVAL;
  uint64_t v = 0;
  switch (what) {
    case PC_KEYSET_DEVICE_BYTES:
      v = (uint64_t)ks->nkeys * (ks->mode ? 2 : 1) * ks->key_words * 4;
      break;
    case PC_KEYSET_KEY_BYTES:
      v = (uint64_t)ks->key_words * 4;
      break;
    case PC_KEYSET_GALOIS: {
      if (bytes != 4 || arg >= ks->nkeys) return PC_EINVAL;
      memcpy(dst, &ks->galois[arg], 4);
      return PC_OK;
    }
    case PC_KEYSET_B_POINTER:
      if (arg >= ks->nkeys) return PC_EINVAL;
      v = (uint64_t)(uintptr_t)ks->b_of(arg);
      break;
    default:
      return PC_EINVAL;
  }
  if (bytes != 8) return PC_EINVAL;
  memcpy(dst, &v, 8);
  return PC_OK;
}

int pc_keyswitch_keyset(const pc_params* p, const pc_keyset* ks, const uint32_t* ct, uint32_t batch,
                        const uint32_t* key_idx, uint32_t nsel, uint32_t level, uint32_t* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (p == nullptr || ks == nullptr || key_idx == nullptr || ks->p != p) return PC_EINVAL;
  if (level < 1 || level > p->L || key_level_of(p, level) != ks->key_level) return PC_EINVAL;
  if (nsel < 1 || nsel > p->max_hoist) return PC_EINVAL;
  const uint32_t* bptr[kMaxKeysPerLaunch];
  const uint32_t* aptr[kMaxKeysPerLaunch];
  uint32_t gal[kMaxKeysPerLaunch];
  uint8_t seeds[kMaxKeysPerLaunch * 32];
  for (uint32_t k = 0; k < nsel; ++k) {
    const uint32_t i = key_idx[k];
    if (i >= ks->nkeys) return PC_EINVAL;
    bptr[k] = ks->b_of(i);
    aptr[k] = ks->a_of(i);
    gal[k] = ks->galois[i];
    memcpy(seeds + 32 * k, &ks->seeds[(size_t)i * 32], 32);
  }
  pc_ks_args a;
  memset(&a, 0, sizeof(a));
  a.ct = ct;
  a.batch = batch;
  a.nkeys = nsel;
  a.evk_b = bptr;
  a.evk_a = ks->mode == PC_KEYSET_FULL ? aptr : nullptr;
  a.seeds = seeds;
  a.galois = gal;
  a.level = level;
  a.out = out;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return pc_keyswitch_ex(p, &a, stream);
}

int pc_chacha_expand(const pc_params* p, const uint8_t* seed, uint32_t d, uint32_t j, uint32_t level, uint32_t* dst,
                     void* stream) {
  if (p == nullptr || seed == nullptr || dst == nullptr || misaligned(dst)) return PC_EINVAL;
  if (level < 1 || level > p->L) return PC_EINVAL;
  if (d >= (uint32_t)beta_of(p, level) || j >= level + p->K) return PC_EINVAL;
  if (p->device < 0) return PC_EDEVICE;
  uint32_t key[8];
  for (int w = 0; w < 8; ++w)
    key[w] = (uint32_t)seed[4 * w] | ((uint32_t)seed[4 * w + 1] << 8) | ((uint32_t)seed[4 * w + 2] << 16) |
             ((uint32_t)seed[4 * w + 3] << 24);
  const uint32_t pi = j < level ? j : p->L + (j - level);
  DeviceGuard g(p->device);
  if (!g.ok) return PC_EDEVICE;
  if (launch_chacha_expand(p, key, d, j, pi, dst, (hipStream_t)stream) != hipSuccess) return PC_EDEVICE;
  return PC_OK;
}

}  // extern "C"
