/*
 * pc.h -- C ABI of the MI355X (gfx950) CKKS hybrid key-switching library.
 *
 * What it computes. The Perseus README ('What's inside') describes a CKKS
 * runtime whose key switching re-creates one half of each key-switching key
 * in its GPU kernels out of a ChaCha12 seed rather than keeping it in memory,
 * and ('Layout') whose device runtime has NTT and key-switching kernels over
 * a 32-bit prime chain (opening paragraph: 32-bit kernels). The arXiv summary
 * page of the Perseus paper (methodology, item (i)) describes that
 * re-creation as ChaCha12 run in counter mode. The pages do not write the
 * algorithm out; this library implements textbook RNS-CKKS hybrid key
 * switching:
 *
 *   ModUp (iNTT, fast base conversion per digit, NTT) -> automorphism ->
 *   inner product with the key (b half read, a half regenerated) ->
 *   ModDown (iNTT of the special limbs, base conversion, NTT, scale by P^-1)
 *   -> add the automorphism of c0.
 *
 * Conventions (readings of what the pages leave open):
 *   - primes: q_0..q_{L-1} then p_0..p_{K-1}, by default every prime r < 2^31
 *     with r = 1 (mod 2N), descending; user chains must be primes in
 *     (2^30, 2^31), r = 1 (mod 2N), pairwise distinct;
 *   - psi_r is the smallest primitive 2N-th root of unity mod r;
 *   - a "limb" is N uint32 canonical residues (< r); polynomials are stored
 *     limb-major, contiguous; evaluation form is natural order,
 *     a_hat[j] = a(psi^(2j+1)) mod r;
 *   - level l = number of active q primes; at level l the digits have
 *     alpha(l) = ceil(l / dnum) primes, D_d = [d alpha, min((d+1) alpha, l)),
 *     beta(l) = ceil(l / alpha) digits; a key used at level l was generated at
 *     level l and has limbs q_0..q_{l-1}, p_0..p_{K-1} (the "key basis");
 *     with partition 1 alpha = ceil(L / dnum) at every level and one key
 *     generated at level L serves every level;
 *   - ciphertext ct = [2][l][N] (c0 then c1), decrypting as c0 + c1 s;
 *   - key b half: [beta][l+K][N] evaluation form (digit, key-basis limb,
 *     position); the a half of digit d, limb j, position i is
 *     (w[2i] + 2^32 w[2i+1]) mod r_j with w the ChaCha stream (12 rounds;
 *     state: "expand 32-byte k", the 32-byte seed as 8 little-endian words,
 *     block counter from 0 in word 12, nonce words (0, d, j)), read in
 *     evaluation form;
 *   - automorphism_idx = Galois element k (odd, < 2N; 1 = none): in evaluation
 *     form out[i] = in[(i k + (k-1)/2) mod N]. It is applied to the ModUp
 *     output (after ModUp, before the inner product) and to c0;
 *   - ModDown uses the floor form (acc - Conv_{P->Q}([acc]_P)) * P^-1.
 *
 * Memory and streams. Every device pointer is a plain device address
 * (hipMalloc or PyTorch memory) on the device the params were created for,
 * 16-byte aligned (the kernels move limbs in 16-byte vectors; a misaligned
 * pointer is rejected with PC_EINVAL); host pointers are marked "host". The
 * caller owns every ciphertext, key, output and workspace buffer; the library
 * owns what its create calls return. Calls enqueue work on `stream` (a
 * hipStream_t; NULL = the null stream) and return without waiting; results
 * are valid once the stream has reached that point. Inputs and outputs must
 * not overlap. The library owns a workspace arena inside pc_params, sized at
 * creation for max_batch ciphertexts and max_hoist keys at any level (the
 * largest of the per-level needs); calls that use it must not run
 * concurrently on different streams for the same pc_params. pc_keyswitch_ex
 * calls that each bring their own workspace may run concurrently on
 * different streams (the constant tables are read-only).
 *
 * Errors. Every entry point validates its arguments on the host before any
 * launch and returns PC_EINVAL (null or misaligned pointer, level outside
 * [1, L], even or out-of-range Galois element, batch above max_batch, ...),
 * PC_EUNSUPPORTED (a shape the kernels do not cover), PC_ENOMEM (allocation at
 * creation) or PC_EDEVICE (a HIP error, including no usable device). No call
 * aborts the process; pc_strerror gives a static message.
 */
#ifndef PC_H
#define PC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pc_params pc_params; /* opaque, library-owned, immutable after creation */

enum {
  PC_OK = 0,
  PC_EINVAL = -1,
  PC_ENOMEM = -2,
  PC_EDEVICE = -3,
  PC_EUNSUPPORTED = -4
};

typedef struct {
  uint32_t log2n;         /* ring degree N = 2^log2n; 12, 16 or 17 */
  uint32_t L;             /* q primes at the top level, >= 1 */
  uint32_t dnum;          /* digits at the top level, 1..6, <= L, with ceil(L / dnum) <= 8 */
  uint32_t K;             /* special primes, 1..8 */
  uint32_t max_batch;     /* most ciphertexts per key-switch call (0 means 1) */
  uint32_t max_hoist;     /* most keys per hoisted call (0 means 1), <= 32 */
  uint32_t chacha_rounds; /* 12 (0 means 12); 20 is accepted for testing against ChaCha20 */
  uint32_t partition;     /* digits below the top level: 0 = alpha(l) = ceil(l / dnum) and keys
                             generated at the ciphertext's level l; 1 = alpha = ceil(L / dnum) at
                             every level (the top-level digits cut at l) and keys generated at
                             level L, whose limbs q_l..q_{L-1} are skipped */
  const uint32_t *primes; /* host; NULL = the descending rule, else L + K primes (q's then p's) */
} pc_params_desc;

/* Parameters, constant tables and the workspace arena (Perseus README,
 * 'Layout': the CUDA-free core holds the parameters and the device runtime
 * one frozen device arena; 'What's inside': programs replay from one device
 * arena whose size is fixed when it starts). Builds the prime chain, psi and every constant table
 * on the host; with device >= 0 also uploads them and allocates the arena on
 * that device. device = -1 builds the host tables only (pc_params_get works;
 * every compute call returns PC_EDEVICE). *out receives a library-owned
 * handle, freed by pc_params_destroy. Errors: PC_EINVAL (null desc or out,
 * L, K or dnum out of range, a bad user prime), PC_EUNSUPPORTED (ring size,
 * digit, special-prime or key limits above), PC_ENOMEM, PC_EDEVICE. */
int pc_params_create(const pc_params_desc *desc, int device, pc_params **out);
/* Frees the tables and the arena of p (Perseus README, Python example under
 * 'Reproduce': a session's resources end with close()). NULL is ignored. */
void pc_params_destroy(pc_params *p);

enum {
  PC_GET_N = 1,               /* uint32: N */
  PC_GET_PRIMES = 2,          /* uint32[L+K] */
  PC_GET_PSI = 3,             /* uint32[L+K] */
  PC_GET_ALPHA = 4,           /* uint32: alpha at level `arg` */
  PC_GET_BETA = 5,            /* uint32: beta at level `arg` */
  PC_GET_WORKSPACE_BYTES = 6, /* uint64: workspace of pc_keyswitch_ex at level `arg` for max_batch x max_hoist */
  PC_GET_DEVICE_TABLE = 7,    /* uint32[N]: forward twiddles psi^bitrev(k) of prime index `arg` (host copy) */
  PC_GET_ARENA_BYTES = 8,     /* uint64: size of the workspace arena (allocated only with a device) */
  PC_GET_LT_WORKSPACE_BYTES = 9 /* uint64: arena bytes pc_linear_transform needs; arg = level | n1 << 8 | n2 << 16 */
};
/* Copies property `what` (argument `arg`) into host memory dst; bytes must be
 * the property's exact size (Perseus README, 'Layout': the core's parameters,
 * here the chain, psi and the digit split). PC_EINVAL for a null pointer, an
 * unknown property, a wrong size or an argument out of range. */
int pc_params_get(const pc_params *p, int what, uint32_t arg, void *dst, size_t bytes);

/* Negacyclic NTT in place (Perseus README, 'Layout': the device runtime's NTT
 * kernels). data is [count][nlimbs][N] (device, coefficients in, natural-order
 * evaluations out); limb z of every one of the count polynomials uses the
 * prime with chain index prime_idx[z] (host array of nlimbs values < L + K).
 * count or nlimbs 0 does nothing. Uses the arena as scratch. PC_EINVAL for a
 * null or misaligned data, a null prime_idx or an index out of range. */
int pc_ntt(const pc_params *p, uint32_t *data, const uint32_t *prime_idx, uint32_t nlimbs, uint32_t count,
           void *stream);
/* Inverse of pc_ntt (Perseus README, 'Layout'), with the N^-1 scale; same
 * arguments and errors. */
int pc_intt(const pc_params *p, uint32_t *data, const uint32_t *prime_idx, uint32_t nlimbs, uint32_t count,
            void *stream);

/* ModUp (Perseus README, 'Layout': the device runtime's key switching; its
 * first step) of c1 ([level][N], evaluation form, device) into ext
 * ([beta][level+K][N], evaluation form, device): for digit d, limbs of D_d are
 * copied from c1, the others are the fast base conversion of the digit
 * ((sum_i [c1_i (Q_d/q_i)^-1]_{q_i} (Q_d/q_i)) mod r_j), taken to evaluation
 * form. Uses the arena. PC_EINVAL for null or misaligned pointers or a level
 * outside [1, L]. */
int pc_modup(const pc_params *p, const uint32_t *c1, uint32_t level, uint32_t *ext, void *stream);

/* One key switch (Perseus README, 'Layout': key switching kernels; 'What's
 * inside': one half of each key re-created in the kernels out of a ChaCha12 seed;
 * arXiv summary page, methodology item (i)): out
 * ([2][level][N], device) from ct ([2][level][N], device) with the key whose
 * b half is evk_b ([beta][kl+K][N], device, kl = the key level) and whose a
 * half is regenerated from evk_seed (32 bytes, host). automorphism_idx is the
 * key's Galois element (1 for relinearisation). Uses the arena. PC_EINVAL
 * for null or misaligned pointers, a null seed, a level outside [1, L], an
 * even Galois element or one >= 2N. */
int pc_keyswitch(const pc_params *p, const uint32_t *ct, const uint32_t *evk_b, const uint8_t *evk_seed,
                 uint32_t level, uint32_t automorphism_idx, uint32_t *out, void *stream);

/* ModDown (Perseus README, 'Layout': the device runtime's key switching; its
 * last step) of one accumulator acc ([level+K][N], evaluation form, device)
 * into out ([level][N], device): (acc - Conv_{P->Q}([acc]_P)) * P^-1 on the q
 * limbs. Uses the arena. PC_EINVAL for null or misaligned pointers or a level
 * outside [1, L]. */
int pc_moddown(const pc_params *p, const uint32_t *acc, uint32_t level, uint32_t *out, void *stream);

/* Batched / hoisted / stored-key key switching (Perseus README, 'Runtime': the
 * primitives are timed at batches k = 1 and 8; 'Layout' and 'What's inside' as
 * for pc_keyswitch). Every ciphertext of the batch is key-switched by every
 * key; ModUp runs once per ciphertext and is shared by all keys (hoisting).
 * The a halves are regenerated from the seeds, or read from evk_a (the
 * stored-key variant, which gives the same bits). PC_EINVAL for null or
 * misaligned pointers, batch or nkeys out of range, a bad Galois element,
 * neither seeds nor evk_a, or a workspace below PC_GET_WORKSPACE_BYTES. */
typedef struct {
  const uint32_t *ct;             /* device [batch][2][level][N] */
  uint32_t batch;                 /* 1..max_batch */
  uint32_t nkeys;                 /* 1..max_hoist */
  const uint32_t *const *evk_b;   /* host array of nkeys device pointers, each [beta(kl)][kl+K][N] with
                                     kl = the key level (level, or L with partition 1) */
  const uint32_t *const *evk_a;   /* NULL (regenerate a from seeds) or host array of nkeys device pointers */
  const uint8_t *seeds;           /* host [nkeys][32]; ignored when evk_a is given */
  const uint32_t *galois;         /* host [nkeys] Galois elements */
  uint32_t level;
  uint32_t *out;                  /* device [nkeys][batch][2][level][N] */
  void *workspace;                /* NULL: the params arena; else device memory of workspace_bytes */
  size_t workspace_bytes;         /* >= PC_GET_WORKSPACE_BYTES for this level (when workspace is given) */
} pc_ks_args;
int pc_keyswitch_ex(const pc_params *p, const pc_ks_args *args, void *stream);

/* Key switching that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments, layouts and results as
 * pc_keyswitch_ex, with workspace NULL and workspace_bytes 0 (PC_EINVAL
 * otherwise): the workspace is a 128 MiB device array inside the library, one
 * copy per GPU, held until the process ends. A call whose workspace need
 * (PC_GET_WORKSPACE_BYTES for its batch and keys) exceeds 128 MiB returns
 * PC_EUNSUPPORTED; at N = 2^16, L = 24, dnum = 4, K = 6 one ciphertext under
 * one or two keys fits. Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, params or threads) race and must be
 * serialised by the caller. No word of the array needs to start at zero. */
int pc_keyswitch_static(const pc_params *p, const pc_ks_args *args, void *stream);

/* Key generation on the GPU (Perseus README, 'What's inside': keys whose a half
 * is regenerated from a ChaCha12 seed). Writes the b half of a key at key level
 * `level` (basis q_0..q_{level-1}, p_0..p_{K-1}, lk = level + K limbs) for
 * Galois element `galois`:
 *   b_d[j] = -a_d[j] s[j] + e_d[j] + g_{d,j} s'[j]  (mod r_j), evaluation form,
 * with a_d the expansion of `seed` (the stream pc_keyswitch regenerates),
 * s' = s^2 for galois 1 (relinearisation) and the automorphism X -> X^galois of
 * s otherwise, and g_{d,j} = [P]_{q_j} on the q-limbs of digit d (digits of
 * `level` under the params' partition), 0 elsewhere.
 *   seed     host, 32 bytes
 *   s_coef   device [lk][N]: the secret's coefficients as residues mod each r_j
 *   e_coef   device [beta][lk][N]: digit d's error coefficients, residues mod r_j
 *   evk_b    device [beta][lk][N] output (beta = digits at `level`)
 * Uses the params' workspace arena ((2 beta + 1) lk N words: the secret, the
 * errors and the transform's scratch; PC_EINVAL if it is smaller). Returns
 * PC_EINVAL for null or misaligned pointers, level outside [1, L] or an even
 * Galois element or one >= 2N, PC_EDEVICE on launch failure. */
int pc_keygen(const pc_params *p, const uint8_t *seed, uint32_t level, uint32_t galois, const uint32_t *s_coef,
              const uint32_t *e_coef, uint32_t *evk_b, void *stream);

/* Homomorphic multiplication around the key switch (Perseus README, Python
 * example under 'Reproduce': squaring a ciphertext is one of the session's
 * ops; the pages leave its steps to the textbook RNS-CKKS product).
 * Ciphertexts are in evaluation form, device buffers owned by the caller; no
 * input may alias an output. All three run on `stream` (hipStream_t or NULL)
 * and return PC_OK, PC_EINVAL for null or misaligned pointers or sizes out of
 * range, PC_EUNSUPPORTED for level - 1 > 64 or 2 batch > 256 (rescale and
 * multiplication only), PC_EDEVICE on launch failure or a host-only params.
 *
 * pc_tensor: per limb i and position, d0 = a0 b0, d1 = a0 b1 + a1 b0,
 * d2 = a1 b1 (mod q_i).
 *   ct_a, ct_b  device [batch][2][level][N]   (1 <= batch <= max_batch)
 *   d           device [batch][3][level][N]   (d0, d1, d2) */
int pc_tensor(const pc_params *p, const uint32_t *ct_a, const uint32_t *ct_b, uint32_t batch, uint32_t level,
              uint32_t *d, void *stream);

/* pc_rescale (Perseus README, 'What's inside': the session's CKKS ops; the
 * textbook rescale): divides by the last prime q_{l-1} (l = level >= 2),
 * rounding to nearest: with x the coefficients of limb l-1 centred into
 * (-q_{l-1}/2, q_{l-1}/2], limb i < l-1 becomes
 * (c_i - NTT_i(x mod q_i)) q_{l-1}^-1 mod q_i.
 *   ct   device [batch][2][level][N]
 *   out  device [batch][2][level-1][N]
 * Uses the params' workspace arena. */
int pc_rescale(const pc_params *p, const uint32_t *ct, uint32_t batch, uint32_t level, uint32_t *out, void *stream);

/* pc_hmult (Perseus README, Python example under 'Reproduce': fhe.square):
 * tensor product, relinearisation of d2 with the key of s^2 (Galois element
 * 1; its a half regenerated from evk_seed as in pc_keyswitch), then
 * pc_rescale: out = rescale(d0 + KS_0(d2), d1 + KS_1(d2)).
 *   ct_a, ct_b  device [batch][2][level][N], 2 <= level <= L
 *   evk_b       device b half of the key (shape as in pc_keyswitch_ex)
 *   evk_seed    host, 32 bytes
 *   out         device [batch][2][level-1][N]
 * Uses the params' workspace arena (sized at create for max_batch at every
 * level). */
int pc_hmult(const pc_params *p, const uint32_t *ct_a, const uint32_t *ct_b, uint32_t batch, const uint32_t *evk_b,
             const uint8_t *evk_seed, uint32_t level, uint32_t *out, void *stream);

/* Double-hoisted baby-step/giant-step linear transform of one ciphertext, the
 * key-switch-heavy stage of a bootstrap (the Perseus README, 'Runtime', times
 * bootstraps with the runtime's primitives). The pages do not write it down;
 * this is the textbook evaluation:
 *   R_0 = (P c0, P c1), R_i = (P phi_{g_i}(c0), 0) + IP(phi_{g_i}(ModUp(c1)), key g_i)
 *       over q_0..q_{l-1}, p_0..p_{K-1} with one shared ModUp (no ModDown);
 *   inner_j = sum_i diag[j][i] R_i;
 *   acc = inner_0 + sum_{j>=1} (phi_{G_j}(inner_j,0), 0)
 *         + IP(phi_{G_j}(ModUp(ModDown(inner_j,1))), key G_j);
 *   out = ModDown(acc).
 * Up to key-switching noise out decrypts to
 * sum_j phi_{G_j}(sum_i diag[j][i] phi_{g_i}(m)). Keys as in pc_keyswitch_ex
 * (b half in device memory, a half regenerated from its seed). All buffers are
 * the caller's; out must not alias ct or diag. Uses the params' workspace arena
 * (PC_EINVAL if it is smaller than PC_GET_LT_WORKSPACE_BYTES for level, n1, n2;
 * a larger max_batch or max_hoist at creation enlarges it). Returns PC_EINVAL for null
 * or misaligned pointers, sizes out of range, an even Galois element or one >= 2N,
 * PC_EDEVICE on launch failure or a host-only params. */
typedef struct {
  const uint32_t *ct;             /* device [2][level][N], evaluation form */
  uint32_t level;                 /* 1..L, with level + K <= 64 */
  uint32_t n1, n2;                /* baby steps 1..8, giant steps 1..32 (identity included) */
  const uint32_t *diag;           /* device [n2][n1][level+K][N]: diagonal (j, i) over the extended basis */
  const uint32_t *const *baby_b;  /* host [n1-1] device pointers: keys of g_1..g_{n1-1} */
  const uint8_t *baby_seeds;      /* host [n1-1][32] */
  const uint32_t *baby_galois;    /* host [n1-1] */
  const uint32_t *const *giant_b; /* host [n2-1] device pointers: keys of G_1..G_{n2-1} */
  const uint8_t *giant_seeds;     /* host [n2-1][32] */
  const uint32_t *giant_galois;   /* host [n2-1] */
  uint32_t *out;                  /* device [2][level][N] */
} pc_lt_args;
int pc_linear_transform(const pc_params *p, const pc_lt_args *args, void *stream);

/* Packed key storage: a key bundle (Perseus README, 'Layout': the server runs
 * on the client's key bundle; 'Runtime': the bootstrap benchmark runs with its
 * keys packed; 'What's inside': one half of each key is re-created from a
 * ChaCha12 seed rather than kept). Reading: a bundle holds nkeys keys
 * of one key level, in one device allocation made at creation -- for each key
 * its b half [beta][kl+K][N], its 32-byte seed and its Galois element (host) --
 * so that the a halves cost 32 bytes each. With PC_KEYSET_FULL the bundle also
 * stores every key's expanded a half beside its b half (twice the device
 * memory: the unpacked form, for comparison); key switches from either form
 * give the same bits. The bundle is library-owned; its keys are written by
 * pc_keyset_set or pc_keyset_keygen and read by pc_keyswitch_keyset. */
typedef struct pc_keyset pc_keyset;
enum { PC_KEYSET_PACKED = 0, PC_KEYSET_FULL = 1 };
/* Creates a bundle (Perseus README, 'Layout': the key bundle; 'Runtime': keys
 * packed) of nkeys (1..256) keys for the key level of ciphertexts at
 * `level` (level itself, or L with partition 1), Galois elements galois
 * (host [nkeys], odd, < 2N, pairwise distinct), on the params' device. Errors:
 * PC_EINVAL (null pointers, sizes, bad or repeated Galois elements, a mode
 * other than the two above), PC_ENOMEM, PC_EDEVICE (host-only params). */
int pc_keyset_create(const pc_params *p, uint32_t level, uint32_t nkeys, const uint32_t *galois, uint32_t mode,
                     pc_keyset **out);
/* Frees the bundle's device allocation (Perseus README, 'Layout': the key
 * bundle). NULL is ignored. */
void pc_keyset_destroy(pc_keyset *ks);
/* Stores key idx (Perseus README, 'Layout': the key bundle): its b half is
 * copied from evk_b (device [beta][kl+K][N]) and its seed (host, 32 bytes)
 * recorded; a FULL bundle also expands the a half on the GPU. PC_EINVAL for a
 * null or misaligned pointer or idx >= nkeys. */
int pc_keyset_set(pc_keyset *ks, uint32_t idx, const uint32_t *evk_b, const uint8_t *seed, void *stream);
/* Generates key idx in place with pc_keygen's equation (Perseus README, 'What's
 * inside'), for the bundle's Galois element of idx: s_coef, e_coef as in
 * pc_keygen. Uses the params' arena. Errors as pc_keygen, and PC_EINVAL for
 * idx >= nkeys. */
int pc_keyset_keygen(pc_keyset *ks, uint32_t idx, const uint8_t *seed, const uint32_t *s_coef, const uint32_t *e_coef,
                     void *stream);
enum {
  PC_KEYSET_DEVICE_BYTES = 1,  /* uint64: device memory the bundle holds */
  PC_KEYSET_KEY_BYTES = 2,     /* uint64: bytes of one b half (and of one stored a half) */
  PC_KEYSET_GALOIS = 3,        /* uint32: Galois element of key `arg` */
  PC_KEYSET_B_POINTER = 4      /* uint64: device address of key `arg`'s b half */
};
/* Copies a property of the bundle (Perseus README, 'Layout': the key bundle)
 * into host memory dst (bytes exact). PC_EINVAL for a null pointer, an
 * unknown property, a wrong size or a key index out of range. */
int pc_keyset_get(const pc_keyset *ks, int what, uint32_t arg, void *dst, size_t bytes);
/* Key switching with keys drawn from a bundle (Perseus README, 'Layout' and
 * 'Runtime'): ciphertexts ct [batch][2][level][N] (device) under the nsel
 * keys key_idx (host [nsel], indices into the bundle), hoisted as in
 * pc_keyswitch_ex, into out [nsel][batch][2][level][N]; a halves regenerated
 * from the bundle's seeds, or read from a FULL bundle. workspace: NULL for the
 * params arena, else device memory of workspace_bytes >=
 * PC_GET_WORKSPACE_BYTES. PC_EINVAL for null or misaligned pointers, an index
 * out of range, nsel above max_hoist, batch above max_batch, a bundle of
 * another params or key level. */
int pc_keyswitch_keyset(const pc_params *p, const pc_keyset *ks, const uint32_t *ct, uint32_t batch,
                        const uint32_t *key_idx, uint32_t nsel, uint32_t level, uint32_t *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Debug / parity (Perseus README, 'What's inside'; arXiv summary page,
 * methodology item (i): the ChaCha12 expander): limb j (key-basis index at
 * `level`) of digit d of the a half regenerated from seed (32 bytes, host):
 * dst ([N], device) canonical mod r_j. PC_EINVAL for a null or misaligned
 * pointer, level out of range, d >= beta or j >= level + K. */
int pc_chacha_expand(const pc_params *p, const uint8_t *seed, uint32_t d, uint32_t j, uint32_t level, uint32_t *dst,
                     void *stream);

/* Measurement support (the pages time their primitives, Perseus README,
 * 'Runtime'). Between pc_profile_begin and pc_profile_end every kernel the
 * library launches for p is bracketed by two hipEvents recorded on the stream
 * it runs on. pc_profile_end waits for those events and writes, per kernel
 * family (stats[k].name is a static string), the number of launches and
 * their summed event-to-event milliseconds; *count receives the number of
 * families written (at most max_stats). Not thread-safe; one profiling window
 * per params at a time. */
typedef struct {
  const char *name;
  uint32_t launches;
  double total_ms;
} pc_kernel_stat;
int pc_profile_begin(const pc_params *p);
int pc_profile_end(const pc_params *p, pc_kernel_stat *stats, uint32_t max_stats, uint32_t *count);

/* Static message for an error code (this ABI's own convention; the pages
 * define none). */
const char *pc_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* PC_H */
