/*
 * fadkv.h -- C ABI of the FAD-KV screening sparse coder with fixed-size dictionary
 * adaptation, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "FAD-KV: Adaptive Dictionary KV Caching for Efficient Reasoning
 * Decoding" (arXiv 2610.37921):
 *   - fadkv_encode: abstract and Figure 1 -- each key/value head vector x is screened against
 *     every atom of its dictionary (scores sigma_j = <d_j, x>), a Top-n pool of the largest
 *     |sigma| is kept, s atoms are chosen inside the pool ("GM" greedy pursuit, or "PL" the s
 *     largest scores; Tables 1-4), and coefficients come from the ridge system of Table 5,
 *     (G_SS + diag(ridge_abs + ridge_rel * G_jj)) c = D_S x.  The relative residual
 *     ||x - D_S^T c|| / ||x|| is compared with delta (Table 5: 0.50 keys, 0.70 values).
 *   - fadkv_adapt: Figure 2 -- vectors whose error exceeds delta overwrite an inactive atom
 *     with their own direction instead of growing the dictionary, so N never changes.
 *   - fadkv_reconstruct: the stored sparse code turned back into a vector (abstract).
 *
 * Conventions shared by every call
 *   - Layout.  A "dictionary set" holds num_dicts independent dictionaries; dictionary t of a
 *     model is 2*layer + 0 for keys and 2*layer + 1 for values (delta is chosen by parity).
 *     atoms are row-major [num_dicts][N][d]; vectors X are [num_dicts][M][d] with the rows of
 *     each dictionary in (head, sequence, token) order -- that order is the commit order of
 *     fadkv_adapt.  Codes are [num_dicts][M][s] (idx int32, coef float) plus relerr float and
 *     flags uint8 per vector.  All these are DEVICE pointers, caller-owned; the library keeps
 *     no pointer after a call returns.
 *   - dtypes.  atoms and X share one storage dtype: FADKV_F32, FADKV_F16 or FADKV_BF16.
 *     Scores multiply in that dtype and accumulate in fp32; everything after the screening
 *     (pool scores, Cholesky, residual) is fp32; new atoms are normalised in fp64 and rounded
 *     to the storage dtype (round to nearest even).
 *   - Limits.  d in {64, 128}; 1 <= N <= 65535; 1 <= s <= n <= min(N, 512); s <= 32;
 *     1 <= num_dicts; 0 <= M and num_dicts * M < 2^31 (every accepted size runs: kernels whose
 *     grid grows with the number of vectors are launched in chunks).  atoms, X and X_hat must be 16-byte
 *     aligned, the other arrays 4-byte aligned (flags: any alignment).
 *   - Streams.  Every call only enqueues work on `stream` (0 = the null stream) and never
 *     synchronises.  On one stream, encode of step t+1 sees adapt of step t.  Calls are
 *     capturable into HIP graphs (no memset or allocation is enqueued).
 *   - Memory.  The calls allocate nothing.  Scratch space is the caller's `workspace`, sized
 *     by fadkv_workspace_bytes; one workspace may be reused by consecutive calls on one stream.
 *   - Errors.  Arguments are checked on the host before anything is enqueued; a bad argument
 *     returns a negative fadkv_status and launches nothing.  A failed launch returns
 *     FADKV_ERR_HIP.  Per-vector outcomes (trigger, replacement, exhaustion, non-finite
 *     input) are reported in flags, never as a status.
 *   - Threads.  Calls on disjoint buffers may run concurrently from several host threads.
 */
#ifndef FADKV_H
#define FADKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FADKV_ABI_VERSION 1

typedef enum {
  FADKV_OK = 0,
  FADKV_ERR_ARG = -1,       /* null or misaligned pointer, negative count, bad parameter */
  FADKV_ERR_DTYPE = -2,     /* unsupported dtype code */
  FADKV_ERR_SHAPE = -3,     /* d, N, n, s or M outside the limits above */
  FADKV_ERR_WORKSPACE = -4, /* workspace null or smaller than fadkv_workspace_bytes */
  FADKV_ERR_HIP = -5,       /* a HIP runtime call or kernel launch failed */
  FADKV_ERR_SCRATCH = -6    /* fadkv_encode_noalloc: the call needs more than its static
                               scratch (FADKV_NOALLOC_SCRATCH_BYTES) */
} fadkv_status;

typedef enum { FADKV_F32 = 0, FADKV_F16 = 1, FADKV_BF16 = 2 } fadkv_dtype;

/* Support rule inside the pool (Tables 1-4 name both; the pages do not define them):
 * GM = s greedy steps, each taking the pool atom of largest |sigma_j - sum_m G_jm c_m|
 *      (ties to the lowest atom index) and re-solving the ridge system;
 * PL = the s pool atoms of largest |sigma| (ties to the lowest index), one ridge solve. */
typedef enum { FADKV_SELECT_GM = 0, FADKV_SELECT_PL = 1 } fadkv_select;

/* flags byte per vector */
#define FADKV_FLAG_TRIGGER 0x01u   /* relative error > delta                          */
#define FADKV_FLAG_REPLACED 0x02u  /* adapt wrote this vector's direction into an atom */
#define FADKV_FLAG_EXHAUSTED 0x04u /* triggered but no inactive atom was left          */
#define FADKV_FLAG_NONFINITE 0x08u /* input held NaN/Inf: empty code, relerr = NaN     */

typedef struct {
  int32_t num_dicts; /* independent dictionaries in the set                       */
  int32_t N;         /* atoms per dictionary (fixed for the life of the set)      */
  int32_t d;         /* head_dim                                                   */
  int32_t dtype;     /* fadkv_dtype of atoms (and of X)                            */
  void *atoms;       /* device [num_dicts][N][d]; only fadkv_adapt writes it       */
  uint32_t *usage;   /* device [num_dicts][N]; committed codes per atom; only
                        fadkv_adapt writes it (start from zeros)                   */
} fadkv_dict;

typedef struct {
  int32_t n;         /* candidate-pool size (Table 5: 256, or 512 for 8B models)   */
  int32_t s;         /* sparsity (Table 5: 8, or 16 for 8B models)                  */
  float ridge_abs;   /* Table 5: 1e-4                                              */
  float ridge_rel;   /* Table 5: 0.20                                              */
  float delta_key;   /* Table 5: 0.50, used by even dictionaries                    */
  float delta_value; /* Table 5: 0.70, used by odd dictionaries                     */
  uint32_t tau_c;    /* atom inactive iff usage < tau_c (and unselected this step);
                        1 = never referenced by a committed code                    */
  int32_t select;    /* fadkv_select                                               */
} fadkv_params;

typedef struct {
  int32_t *idx;   /* device [num_dicts][M][s]: atom indices in selection order, -1 = empty */
  float *coef;    /* device [num_dicts][M][s]: coefficients, 0 for empty slots             */
  float *relerr;  /* device [num_dicts][M]: ||x - x_hat|| / ||x|| (0 for x = 0)            */
  uint8_t *flags; /* device [num_dicts][M]: FADKV_FLAG_* bits                              */
} fadkv_codes;

/* Bytes of device workspace that fadkv_encode and fadkv_adapt need for M vectors per
 * dictionary (the larger of the two; one buffer serves both).  Writes *bytes and returns
 * FADKV_OK, or a negative status if the shapes are outside the limits. */
int fadkv_workspace_bytes(const fadkv_dict *dict, const fadkv_params *params, int64_t M,
                          size_t *bytes);

/* Encode M vectors per dictionary (abstract; Figure 1; Table 5).
 *   X: device [num_dicts][M][d] in dict->dtype.
 *   out: codes written for every vector; flags get TRIGGER or NONFINITE only.
 * A vector of zeros gets the empty code and relerr 0.  The dictionary is read only. */
int fadkv_encode(const fadkv_dict *dict, const fadkv_params *params, const void *X, int64_t M,
                 const fadkv_codes *out, void *workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* fadkv_encode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and the same
 * results as fadkv_encode, with the candidate pools kept in a static device array of
 * FADKV_NOALLOC_SCRATCH_BYTES instead of a caller workspace.  Each GPU the library runs on
 * holds its own copy of that array until the process ends; the call uses the copy of the
 * current device (make the device of `stream` current before calling).  It allocates
 * nothing, enqueues no memset and never synchronises.
 *   Limit: the call needs fadkv_workspace_bytes(dict, params, M) <= FADKV_NOALLOC_SCRATCH_BYTES
 *   (about num_dicts * M * (6 n + 1) bytes; e.g. 56 x 256 vectors at n = 256, or 64 x 512 at
 *   n = 512); larger calls return FADKV_ERR_SCRATCH and launch nothing.
 *   Concurrency: every call on one GPU shares that GPU's array, so calls that overlap on one
 *   GPU (two streams, two host threads) race; serialise them (one stream) or use fadkv_encode
 *   with separate workspaces.  The array keeps the last call's contents; nothing in it needs
 *   to start at zero. */
#define FADKV_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int fadkv_encode_noalloc(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                         int64_t M, const fadkv_codes *out, hipStream_t stream);

/* The two stages of fadkv_encode, for callers that want the candidate pool itself (e.g. to
 * measure how much of a full pursuit's support it recalls, Figure 1b) or to time each stage.
 *
 * fadkv_screen -- abstract and Figure 1: scores sigma_j = <d_j, x> of every atom and the pool
 * of the n largest |sigma| (ties to the lowest index).
 *   pool_idx:   device uint16 [num_dicts][M][n], the pool's atom indices (unordered set);
 *   pool_score: device float  [num_dicts][M][n], sigma of each pool atom (fp32 accumulation);
 *   vstatus:    device uint8  [num_dicts][M], 0 = encoded, 1 = zero vector, 2 = non-finite
 *               input (pool rows of status 1 and 2 are left unwritten).
 * Needs no workspace. */
int fadkv_screen(const fadkv_dict *dict, const fadkv_params *params, const void *X, int64_t M,
                 uint16_t *pool_idx, float *pool_score, uint8_t *vstatus, hipStream_t stream);

/* fadkv_select_support -- Tables 1-5: the s-atom support inside each pool (GM or PL), the
 * ridge coefficients and the relative residual against delta, from fadkv_screen's outputs
 * (same dict, params, X and M).  Writes `out` exactly as fadkv_encode does. */
int fadkv_select_support(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                         int64_t M, const uint16_t *pool_idx, const float *pool_score,
                         const uint8_t *vstatus, const fadkv_codes *out, hipStream_t stream);

/* Full-dictionary greedy yardstick: the "full-OMP atoms" Figure 1b compares the screened pool
 * against, and the Cost 1.00 reference of Table 4.  The same greedy steps as GM (largest
 * |rho_j| = |<d_j, x - D_S^T c>|, ties to the lowest index, chosen atoms excluded, the ridge
 * system of Table 5 re-solved at every step) with every atom of the dictionary a candidate
 * instead of the Top-n pool; params->n and params->select are not used.  Writes `out` as
 * fadkv_encode does (same zero and non-finite handling, same trigger against delta).
 * Launches 1 + 2 s kernels on `stream`.  workspace: fadkv_omp_workspace_bytes(), 256-byte
 * aligned, owned by the caller; X: device [num_dicts][M][d], 16-byte aligned. */
int fadkv_omp_workspace_bytes(const fadkv_dict *dict, const fadkv_params *params, int64_t M,
                              size_t *bytes);
int fadkv_encode_omp(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                     int64_t M, const fadkv_codes *out, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Commit one step's codes and apply fixed-size adaptation (Figure 2), per dictionary:
 *   1. usage[j] += 1 for every atom of every non-triggering code;
 *   2. candidates = atoms with usage < tau_c that no code of this step selected, ordered by
 *      (usage, atom index);
 *   3. the k-th triggering row (row order) takes the k-th candidate j: atom j becomes
 *      x/||x|| rounded to the storage dtype, usage[j] = 1, and the row's code becomes the
 *      single atom j with coefficient <d_j, x> / ((1 + ridge_rel) ||d_j||^2 + ridge_abs)
 *      (relerr recomputed, flag REPLACED);
 *   4. triggering rows beyond the candidates keep their code, commit its usage and get flag
 *      EXHAUSTED.
 * X and codes must be those of the fadkv_encode call of this step (codes is updated in
 * place).  replaced: device [num_dicts][M] int32, the overwritten atom per row or -1.
 * atoms and usage are updated in place; N never changes. */
int fadkv_adapt(const fadkv_dict *dict, const fadkv_params *params, const void *X, int64_t M,
                const fadkv_codes *codes, int32_t *replaced, void *workspace,
                size_t workspace_bytes, hipStream_t stream);

/* Append-only growth: the contrast the abstract draws (an adaptive dictionary that only ever
 * appends keeps growing during generation; FAD-KV, abstract and Fig. 3a), offered to measure it.  Same as fadkv_adapt except where a
 * triggering row's new atom goes: dictionary t uses slots [0, n_atoms[t]) of its capacity N
 * (dict->N; unused slots must hold zeros: they score 0 and are never selected), and its k-th
 * triggering row (row order) writes round(x/||x||) to slot n_atoms[t] + k while slots remain,
 * is re-coded onto it (flag REPLACED, replaced[m] = the slot) and leaves every existing atom
 * untouched; rows past the capacity keep their code, commit its usage and get flag EXHAUSTED.
 * n_atoms: device int32 [num_dicts], read and advanced in place (values clamped to [0, N]).
 * Non-triggering rows commit usage exactly as in fadkv_adapt; tau_c is not used. */
int fadkv_adapt_append(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                       int64_t M, const fadkv_codes *codes, int32_t *replaced, int32_t *n_atoms,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* x_hat[t][m] = sum over non-empty slots k of coef[t][m][k] * atoms[t][idx[t][m][k]],
 * written as out_dtype (fp32 accumulation; 16-bit outputs rounded to nearest even).
 * idx entries must be -1 or in [0, N). */
int fadkv_reconstruct(const fadkv_dict *dict, const int32_t *idx, const float *coef, int32_t s,
                      int64_t M, void *X_hat, int32_t out_dtype, hipStream_t stream);

/* ---- decode attention over the codes ------------------------------------------------------
 * The consumer of the encoder's output.  The abstract stores every token's key and value as a
 * sparse combination of atoms, so a decode query meets the cached keys through the atoms:
 * <q, k_t> = sum_k cK[t][k] <q, d^K_{iK[t][k]}> needs q . D_K^T once per query and s gathers
 * per token, and the weighted values sum to w . D_V with w the softmax weights scattered onto
 * the atoms.  The pages give no formula for this step; the definition taken is standard scaled
 * softmax attention over the rebuilt tokens:
 *   out[r][g] = sum_{t < len[r]} p_t v_t,  p = softmax_t(scale * <q[r][g], k_t>),
 *   k_t = sum_k cK[r][t][k] d^K_{iK[r][t][k]}, v_t = sum_k cV[r][t][k] d^V_{iV[r][t][k]},
 * and out[r][g] = 0 for a row without tokens.
 *
 * Layer `layer` takes its keys from dictionary 2*layer of `dict` and its values from 2*layer+1
 * (0 <= layer, 2*layer + 1 < num_dicts).  Rows r < R are (KV head, sequence) pairs:
 *   k_idx, v_idx  device int32 [R][T][s]  atom per slot; -1 (or anything outside [0, N)) = empty
 *   k_coef, v_coef device fp32 [R][T][s]
 *   lens          device int32 [R]        cached tokens of the row (clamped to [0, T])
 *   q             device [R][G][d] in the dictionary dtype, 16-byte aligned; G query heads
 *                 share row r's keys and values (1 <= G <= 64)
 *   out           device fp32 [R][G][d], overwritten
 *   scale         finite (e.g. 1/sqrt(d))
 * 1 <= s <= 32, N <= 16384, 0 <= R <= 2^22, T >= 0, R*G <= 2^24 (the kernels' grids).
 * Workspace: at least fadkv_attend_workspace_bytes() bytes, 256-byte aligned, caller-owned (it
 * holds q . D_K^T, then the atom weights, fp32 [R*G][N], and partial outputs per range of 128
 * atoms, fp32 [ceil(N/128)][R*G][d]).  Checked synchronously; nothing is launched on error.
 * fp32 throughout after the 16-bit products.  Determinism: for N <= 13311 the value weights
 * are accumulated exactly as 64-bit fixed point, so out is bitwise reproducible; for larger N
 * they are accumulated with fp32 LDS atomics, whose order varies, so the last bits of out may
 * differ between runs. */
int fadkv_attend_workspace_bytes(const fadkv_dict *dict, int64_t R, int32_t G, size_t *bytes);
int fadkv_attend(const fadkv_dict *dict, int32_t layer, int32_t s, const int32_t *k_idx,
                 const float *k_coef, const int32_t *v_idx, const float *v_coef,
                 const int32_t *lens, int64_t R, int32_t T, const void *q, int32_t G,
                 float scale, float *out, void *workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *fadkv_status_string(int status);

/* FADKV_ABI_VERSION of the built library. */
int fadkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FADKV_H */
