// PL support selection (FAD-KV Tables 1-4, "PL"): the s pool atoms of largest |sigma| (ties to
// the lowest atom index), one ridge solve (G_SS + diag(ridge_abs + ridge_rel G_jj)) c = sigma_S
// (Table 5), the residual r = x - D_S^T c and its relative norm against delta.
//
// One wave per vector, no barrier.  The pool's scores are spread over the lanes (entry
// lane + 64 q); s rounds of a wave-wide argmax pick the support in rank order.  Lanes then
// compute the lower triangle of G_SS (one entry per lane and round, from the two stored rows)
// into the wave's LDS block.  The Cholesky factor is built one row per step: lanes i < k carry
// the right-hand side of L_{<k} l = G_{<k,k} while each l_m is broadcast, so lane i keeps row i
// of L and column i of L in registers; the two triangular solves run across lanes the same way.
#include "common.h"
#include "kernels.h"

namespace fadkv {

namespace {

constexpr int PL_WAVES = 4;
constexpr int PL_QMAX = 8;   // pool entries per lane (n <= 512)

template <int DT, int D>
__device__ __forceinline__ float pl_row_dot(const uint8_t *a, const uint8_t *b) {
  constexpr int CPR = D * Elem<DT>::bytes / 16;
  const uint4 *pa = reinterpret_cast<const uint4 *>(a);
  const uint4 *pb = reinterpret_cast<const uint4 *>(b);
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < CPR; ++c) {
    const uint4 u = pa[c], v = pb[c];
    if constexpr (DT == DT_F32) {
      s0 = fmaf(__uint_as_float(u.x), __uint_as_float(v.x), s0);
      s1 = fmaf(__uint_as_float(u.y), __uint_as_float(v.y), s1);
      s0 = fmaf(__uint_as_float(u.z), __uint_as_float(v.z), s0);
      s1 = fmaf(__uint_as_float(u.w), __uint_as_float(v.w), s1);
    } else {
      s0 = dot2<DT>(u.x, v.x, s0);
      s1 = dot2<DT>(u.y, v.y, s1);
      s0 = dot2<DT>(u.z, v.z, s0);
      s1 = dot2<DT>(u.w, v.w, s1);
    }
  }
  return s0 + s1;
}

}  // namespace

template <int DT, int D, int SMAX>
__global__ __launch_bounds__(PL_WAVES * 64) void select_pl_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int N, int M, size_t G,
    int n, int s, float ridge_abs, float ridge_rel, float delta_key, float delta_value,
    const uint16_t *__restrict__ pool_idx, const float *__restrict__ pool_sig,
    const uint8_t *__restrict__ vstat, int32_t *__restrict__ out_idx,
    float *__restrict__ out_coef, float *__restrict__ out_relerr,
    uint8_t *__restrict__ out_flags, size_t base) {
  constexpr int ROWB = D * Elem<DT>::bytes;
  constexpr int PER = D / 64;
  __shared__ float s_G[PL_WAVES][SMAX * SMAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t gv = base + (size_t)blockIdx.x * PL_WAVES + wave;
  if (gv >= G) return;
  const int dict = (int)(gv / (size_t)M);
  const uint8_t st = vstat[gv];
  if (st != VS_NORMAL) {
    if (lane < s) {
      out_idx[gv * s + lane] = -1;
      out_coef[gv * s + lane] = 0.f;
    }
    if (lane == 0) {
      out_relerr[gv] = st == VS_ZERO ? 0.f : __builtin_nanf("");
      out_flags[gv] = st == VS_ZERO ? 0 : FLAG_NONFINITE;
    }
    return;
  }
  const uint8_t *dict_atoms = atoms + (size_t)dict * N * ROWB;
  float *Gw = s_G[wave];

  // pool entries of this lane: |sigma| bits (-1 = absent or taken), signed sigma, atom
  int key[PL_QMAX], atom[PL_QMAX];
  float sg[PL_QMAX];
#pragma unroll
  for (int q = 0; q < PL_QMAX; ++q) {
    const int e = lane + 64 * q;
    key[q] = -1;
    atom[q] = 0x7fffffff;
    sg[q] = 0.f;
    if (e < n) {
      const float v = pool_sig[gv * n + e];
      float a = fabsf(v);
      a = a != a ? 0.f : a;   // a NaN score (non-finite atoms) ranks as 0
      key[q] = __float_as_int(a);
      const int j = pool_idx[gv * n + e];
      atom[q] = j < N ? j : N - 1;
      sg[q] = v;
    }
  }

  // s rounds of argmax: lane k keeps the k-th atom and its score
  int my_atom = 0;
  float my_sig = 0.f;
#pragma unroll
  for (int k = 0; k < SMAX; ++k) {
    if (k < s) {
      int bk = -1, bj = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < PL_QMAX; ++q) {
        const bool better = key[q] > bk || (key[q] == bk && key[q] >= 0 && atom[q] < bj);
        bk = better ? key[q] : bk;
        bj = better ? atom[q] : bj;
      }
      const int wk = wave_max_nonneg_bits(bk);
      int wj = wave_min_i32(bk == wk ? bj : 0x7fffffff);
      // a pool that repeats atoms can run out before s picks (the screening never writes one,
      // but the call accepts any pool): the index must still name a row of the dictionary
      wj = wj < N ? wj : N - 1;
      float got = 0.f;
      bool mine = false;
#pragma unroll
      for (int q = 0; q < PL_QMAX; ++q) {
        const bool hit = key[q] >= 0 && atom[q] == wj;
        got = hit ? sg[q] : got;
        mine = mine || hit;
        key[q] = hit ? -1 : key[q];
      }
      const unsigned long long owner = __builtin_amdgcn_ballot_w64(mine);
      const int ol = owner ? (int)__ffsll((long long)owner) - 1 : 0;
      const float sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(got), ol));
      if (lane == k) {
        my_atom = wj;
        my_sig = sk;
      }
    }
  }

  // lower triangle of G_SS: entry e = r (r + 1) / 2 + c, c <= r
  const int ne = s * (s + 1) / 2;
  for (int e0 = 0; e0 < ne; e0 += 64) {   // wave-uniform rounds; shuffles with every lane on
    const int e = e0 + lane;
    const int ee = e < ne ? e : 0;
    int r = (int)((sqrtf(8.f * (float)ee + 1.f) - 1.f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= ee) ++r;
    while (r * (r + 1) / 2 > ee) --r;
    const int c = ee - r * (r + 1) / 2;
    const int ar = __shfl(my_atom, r), ac = __shfl(my_atom, c);
    if (e < ne)
      Gw[r * SMAX + c] = pl_row_dot<DT, D>(dict_atoms + (size_t)ar * ROWB,
                                           dict_atoms + (size_t)ac * ROWB);
  }
  // the entries written by other lanes of this wave are read below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  // Cholesky, one row per step (lane i: Lrow = L[i][0..i-1], dg = L[i][i]); row k of L then
  // overwrites row k of G in LDS (that row is not read again) for the back substitution
  float Lrow[SMAX];
#pragma unroll
  for (int m = 0; m < SMAX; ++m) Lrow[m] = 0.f;
  float dg = 1.f;
#pragma unroll 8
  for (int k = 0; k < SMAX; ++k) {
    if (k < s) {
      float g = lane < k ? Gw[k * SMAX + lane] : 0.f;
      const float gkk = Gw[k * SMAX + k];
      float mine = 0.f, sumsq = 0.f;
#pragma unroll
      for (int m = 0; m < SMAX; ++m) {
        if (m < k) {
          const float lm = __shfl(g, m) / __shfl(dg, m);
          sumsq = fmaf(lm, lm, sumsq);
          if (lane == m) mine = lm;
          if (lane == k) Lrow[m] = lm;
          if (lane > m) g = fmaf(-Lrow[m], lm, g);
        }
      }
      const float lkk = sqrtf(fmaxf(fmaf(gkk, 1.f + ridge_rel, ridge_abs) - sumsq, 1e-30f));
      if (lane < k) Gw[k * SMAX + lane] = mine;
      if (lane == k) dg = lkk;
    }
  }
  // y = L^{-1} sigma_S, then c = L^{-T} y (lane i ends with c_i)
  float b = lane < s ? my_sig : 0.f, y = 0.f;
#pragma unroll
  for (int m = 0; m < SMAX; ++m) {
    if (m < s) {
      const float ym = __shfl(b, m) / __shfl(dg, m);
      if (lane == m) y = ym;
      if (lane > m) b = fmaf(-Lrow[m], ym, b);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float c = 0.f;
#pragma unroll
  for (int m = SMAX - 1; m >= 0; --m) {
    if (m < s) {
      const float cm = __shfl(y, m) / __shfl(dg, m);
      if (lane == m) c = cm;
      if (lane < m) y = fmaf(-Gw[m * SMAX + lane], cm, y);
    }
  }

  // r = x - D_S^T c, e = ||r|| / ||x||
  const uint8_t *xr = X + gv * ROWB;
  float rv[PER], xx = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    rv[p] = elem_f<DT>(xr, lane + 64 * p);
    xx = fmaf(rv[p], rv[p], xx);
  }
#pragma unroll
  for (int m = 0; m < SMAX; ++m) {
    if (m < s) {
      const float cm = __shfl(c, m);
      const uint8_t *row = dict_atoms + (size_t)__shfl(my_atom, m) * ROWB;
#pragma unroll
      for (int p = 0; p < PER; ++p) rv[p] = fmaf(-cm, elem_f<DT>(row, lane + 64 * p), rv[p]);
    }
  }
  float rr = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) rr = fmaf(rv[p], rv[p], rr);
  rr = wave_sum(rr);
  xx = wave_sum(xx);
  if (lane < s) {
    out_idx[gv * s + lane] = my_atom;
    out_coef[gv * s + lane] = c;
  }
  if (lane == 0) {
    const float e = sqrtf(rr / xx);
    out_relerr[gv] = e;
    out_flags[gv] = e > ((dict & 1) ? delta_value : delta_key) ? FLAG_TRIGGER : 0;
  }
}

hipError_t launch_select_pl(int dtype, int d, const void *atoms, const void *X, int num_dicts,
                            int N, int M, int n, int s, float ridge_abs, float ridge_rel,
                            float delta_key, float delta_value, const uint16_t *pool_idx,
                            const float *pool_sig, const uint8_t *vstat, int32_t *idx,
                            float *coef, float *relerr, uint8_t *flags, hipStream_t stream) {
  const size_t G = (size_t)num_dicts * M;
  const size_t blocks = (G + PL_WAVES - 1) / PL_WAVES;
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
  for (size_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
    const dim3 grid((unsigned)nb), block(PL_WAVES * 64);
#define L(DT, D, SM)                                                                              \
  hipLaunchKernelGGL((select_pl_kernel<DT, D, SM>), grid, block, 0, stream, A, Xb, N, M, G, n, s, \
                     ridge_abs, ridge_rel, delta_key, delta_value, pool_idx, pool_sig, vstat, idx, \
                     coef, relerr, flags, b0 * PL_WAVES)
#define LS(DT, D) do { if (s <= 8) L(DT, D, 8); else if (s <= 16) L(DT, D, 16); else L(DT, D, 32); } while (0)
#define LD(DT) do { if (d == 64) LS(DT, 64); else LS(DT, 128); } while (0)
    if (dtype == DT_F32) LD(DT_F32);
    else if (dtype == DT_F16) LD(DT_F16);
    else LD(DT_BF16);
#undef LD
#undef LS
#undef L
  }
  return hipGetLastError();
}

}  // namespace fadkv
