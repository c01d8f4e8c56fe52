// Host-side launchers of the FAD-KV kernels (internal to libfadkv; see include/fadkv.h for the
// public C ABI).  Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fadkv {

hipError_t launch_score_topn(int dtype, int d, const void *atoms, const void *X, int num_dicts,
                             int N, int M, int n, uint16_t *pool_idx, float *pool_sig,
                             uint8_t *vstat, hipStream_t stream);

// GM: greedy pursuit inside the pool (one workgroup per vector)
hipError_t launch_select(int dtype, int d, const void *atoms, const void *X, int num_dicts, int N,
                         int M, int n, int s, float ridge_abs, float ridge_rel,
                         float delta_key, float delta_value, const uint16_t *pool_idx,
                         const float *pool_sig, const uint8_t *vstat, int32_t *idx, float *coef,
                         float *relerr, uint8_t *flags, hipStream_t stream);

// PL: the s largest |sigma| of the pool, one solve (one wave per vector)
hipError_t launch_select_pl(int dtype, int d, const void *atoms, const void *X, int num_dicts,
                            int N, int M, int n, int s, float ridge_abs, float ridge_rel,
                            float delta_key, float delta_value, const uint16_t *pool_idx,
                            const float *pool_sig, const uint8_t *vstat, int32_t *idx,
                            float *coef, float *relerr, uint8_t *flags, hipStream_t stream);

hipError_t launch_adapt(int dtype, int d, void *atoms, uint32_t *usage, const void *X, int num_dicts,
                        int N, int M, int s, float ridge_abs, float ridge_rel, uint32_t tau_c,
                        int32_t *idx, float *coef, float *relerr, uint8_t *flags,
                        int32_t *replaced, uint8_t *touched, int touched_stride, int32_t *rank,
                        int32_t *cand, int32_t *ccount, int32_t *n_atoms, hipStream_t stream);

hipError_t launch_reconstruct(int dtype, int d, const void *atoms, const int32_t *idx,
                              const float *coef, int num_dicts, int N, int M, int s, void *out,
                              int out_dtype, hipStream_t stream);

// decode attention over the codes: qd = Q D_K^T (and out = 0), per-row softmax scattering the
// value weights onto the atoms (in place over qd), out += weights . D_V
hipError_t launch_attend(int dtype, int d, const void *dictK, const void *dictV, int N, int s,
                         const int32_t *k_idx, const float *k_coef, const int32_t *v_idx,
                         const float *v_coef, const int32_t *lens, int R, int T, const void *q,
                         int G, float scale, float *out, float *ws, hipStream_t stream);

// full-dictionary greedy yardstick: init, then per step a correlation sweep and an update
struct OmpArgs {
  const void *atoms;
  const void *X;
  int num_dicts, N, M, s;
  float ridge_abs, ridge_rel, delta_key, delta_value;
  uint8_t *status;   // [G] vector class
  int32_t *jstar;    // [G] atom chosen by the current step
  int32_t *S;        // [G][s] chosen atoms, selection order
  float *L;          // [G][s][s] Cholesky rows
  float *sig;        // [G][s] <d_S[i], x>
  uint8_t *R;        // [G] residual rows (omp_residual_row_bytes each)
  int32_t *idx;
  float *coef;
  float *relerr;
  uint8_t *flags;
};
size_t omp_residual_row_bytes(int dtype, int d);
hipError_t launch_omp(int dtype, int d, const OmpArgs &a, hipStream_t stream);

}  // namespace fadkv
