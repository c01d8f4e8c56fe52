// Support selection inside the candidate pool, ridge coefficients and relative residual.
//
// One workgroup per vector; thread t owns pool entry t: its atom row stays in registers
// (packed 16-bit pairs or fp32), together with its score sigma_t and, for GM, its row of
// W = G_{P,S} L^{-T}, where L L^T = G_SS + diag(ridge_abs + ridge_rel * G_jj) (Table 5).
//
// GM (greedy pursuit in the pool).  With y = L^{-1} sigma_S the ridge coefficients are
// c = L^{-T} y, and the correlation of pool atom j with the residual of the current code is
// rho_j = sigma_j - G_{j,S} c = sigma_j - W_j . y.  Step k picks j* = argmax |rho_j| over the
// pool atoms not yet chosen (ties to the lowest atom index), then
//   l      = W_{j*, 0..k-1}                 (new Cholesky row: L^{-1} G_{S,j*})
//   L_kk   = sqrt((1 + ridge_rel) G_j*j* + ridge_abs - |l|^2)
//   y_k    = (sigma_j* - l . y) / L_kk
//   W_{:,k} = (G_{P,j*} - W_{:,0..k-1} l) / L_kk,     rho -= W_{:,k} y_k
// which needs one pool-wide column G_{P,j*} = D_P d_j* per step (skipped after the last
// step) and O(k) work per pool atom.  At the end c = L^{-T} y by back substitution.
// PL takes the s largest |sigma| of the pool the same way (no rho update) and solves once.
// Finally r = x - D_S^T c is formed from the chosen rows and e = ||r|| / ||x||.
//
// Each step costs two workgroup barriers: (1) after every wave has published its local
// argmax (wave reduction through DPP), (2) after the winner has published its W row, score
// and squared norm.  The winning row itself is read by every wave through the scalar cache.
// The LDS slots are double-buffered by step parity, so no third barrier is needed before they
// are rewritten.
#include "common.h"
#include "kernels.h"

namespace fadkv {

namespace {
constexpr int MAX_THREADS = 512;
constexpr int MAX_WAVES = MAX_THREADS / 64;
}  // namespace

template <int DT, int D> struct RowWords {
  static constexpr int NW = DT == DT_F32 ? D : D / 2;   // 32-bit words per atom row
  static constexpr int ROWB = D * Elem<DT>::bytes;
};

// Dot product of the thread's row with a row every lane reads at the same address.  The address
// is wave-uniform and the atoms are read-only in this kernel, so the compiler fetches that row
// with scalar loads and feeds it to v_dot2 as the scalar operand: no LDS broadcast and no
// vector registers for the shared row.
template <int DT, int NW>
__device__ __forceinline__ float row_dot_uniform(const uint32_t (&a)[NW],
                                                 const uint32_t *__restrict__ row) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int q = 0; q < NW; q += 2) {
    if constexpr (DT == DT_F32) {
      s0 = fmaf(__uint_as_float(a[q]), __uint_as_float(row[q]), s0);
      s1 = fmaf(__uint_as_float(a[q + 1]), __uint_as_float(row[q + 1]), s1);
    } else {
      s0 = dot2<DT>(a[q], row[q], s0);
      s1 = dot2<DT>(a[q + 1], row[q + 1], s1);
    }
  }
  return s0 + s1;
}

template <int DT, int NW>
__device__ __forceinline__ float row_self_dot(const uint32_t (&a)[NW]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int q = 0; q < NW; q += 2) {
    if constexpr (DT == DT_F32) {
      s0 = fmaf(__uint_as_float(a[q]), __uint_as_float(a[q]), s0);
      s1 = fmaf(__uint_as_float(a[q + 1]), __uint_as_float(a[q + 1]), s1);
    } else {
      s0 = dot2<DT>(a[q], a[q], s0);
      s1 = dot2<DT>(a[q + 1], a[q + 1], s1);
    }
  }
  return s0 + s1;
}

// element i of a packed row held in LDS
template <int DT> __device__ __forceinline__ float lds_elem(const uint32_t *row, int i) {
  if constexpr (DT == DT_F32) return __uint_as_float(row[i]);
  else return (i & 1) ? hi_f<DT>(row[i >> 1]) : lo_f<DT>(row[i >> 1]);
}

template <int DT, int D, int SMAX>
__global__ __launch_bounds__(MAX_THREADS) void select_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int num_dicts, int N, int M,
    int n, int s, int select, float ridge_abs, float ridge_rel, float delta_key, float delta_value,
    const uint16_t *__restrict__ pool_idx, const float *__restrict__ pool_sig,
    const uint8_t *__restrict__ vstat, int32_t *__restrict__ out_idx, float *__restrict__ out_coef,
    float *__restrict__ out_relerr, uint8_t *__restrict__ out_flags) {
  constexpr int NW = RowWords<DT, D>::NW;
  constexpr int ROWB = RowWords<DT, D>::ROWB;
  __shared__ __attribute__((aligned(16))) uint32_t s_selrow[SMAX][NW];  // chosen rows
  __shared__ float s_x[D];
  __shared__ float s_L[SMAX * SMAX];
  __shared__ float s_y[SMAX], s_c[SMAX], s_sig[SMAX], s_gdiag[SMAX];
  __shared__ float s_l[2][SMAX];
  __shared__ int s_sel[SMAX];
  __shared__ float s_rv[2][MAX_WAVES];
  __shared__ int s_rj[2][MAX_WAVES];
  __shared__ float s_sum[2][MAX_WAVES];

  // With a multiple of 8 dictionaries, workgroup i (dispatched to XCD i % 8) takes a vector of
  // dictionary xcd + 8 * (r / M), r = i / 8: each dictionary's pool rows are gathered through
  // one XCD's L2.
  size_t gv;
  if ((num_dicts & 7) == 0) {
    const size_t r = blockIdx.x / 8;
    const int xcd = blockIdx.x % 8;
    gv = (size_t)(xcd + 8 * (int)(r / (size_t)M)) * M + r % (size_t)M;
  } else {
    gv = blockIdx.x;
  }
  const int dict = (int)(gv / (size_t)M);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const float delta = (dict & 1) ? delta_value : delta_key;

  const uint8_t st = vstat[gv];
  if (st != VS_NORMAL) {
    if (tid < s) {
      out_idx[gv * s + tid] = -1;
      out_coef[gv * s + tid] = 0.f;
    }
    if (tid == 0) {
      out_relerr[gv] = st == VS_ZERO ? 0.f : __builtin_nanf("");
      out_flags[gv] = st == VS_ZERO ? 0 : FLAG_NONFINITE;
    }
    return;
  }

  const uint8_t *dict_atoms = atoms + (size_t)dict * N * ROWB;
  const bool act = tid < n;
  int j = 0x7fffffff;
  float sig = 0.f;
  if (act) {
    const int jj = pool_idx[gv * n + tid];
    j = jj < N ? jj : N - 1;   // the screening kernel writes indices < N; never read past the set
    sig = pool_sig[gv * n + tid];
  }
  // each thread loads its own pool row (all 16-byte loads issued back to back)
  uint32_t w[NW];
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(dict_atoms + (size_t)(act ? j : 0) * ROWB);
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const uint4 v = act ? src[q] : make_uint4(0, 0, 0, 0);
      w[4 * q + 0] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
  }
  const float gself = row_self_dot<DT, NW>(w);   // ||d_j||^2, needed if this row is chosen
  for (int i = tid; i < D; i += blockDim.x) s_x[i] = elem_f<DT>(X + gv * ROWB, i);
  if (tid < SMAX) s_sel[tid] = 0;   // every slot names a valid row even if no thread wins

  const bool gm = select == 0;
  float rho = sig;
  float W[SMAX];
#pragma unroll
  for (int m = 0; m < SMAX; ++m) W[m] = 0.f;
  bool chosen = false;

#pragma unroll
  for (int k = 0; k < SMAX; ++k) {
    if (k < s) {
      const int buf = k & 1;
      // (1) wave argmax of |rho| over unchosen entries, ties to the lowest atom index
      const bool elig = act && !chosen;
      float v = elig ? fabsf(rho) : -1.f;
      v = v != v ? 0.f : v;   // a NaN score (non-finite atoms) ranks as 0, never above real ones
      const float wmax = wave_max_f32(v);
      const unsigned long long hit = __ballot(elig && v == wmax);
      int wj;
      if (__popcll(hit) == 1) wj = __builtin_amdgcn_readlane(j, (int)__ffsll((long long)hit) - 1);
      else wj = wave_min_i32((elig && v == wmax) ? j : 0x7fffffff);
      if (lane == 0) {
        s_rv[buf][wave] = wmax;
        s_rj[buf][wave] = wj;
      }
      __syncthreads();
      float bv = s_rv[buf][0];
      int bj = s_rj[buf][0];
      for (int q = 1; q < nwaves; ++q) {
        const float qv = s_rv[buf][q];
        const int qj = s_rj[buf][q];
        if (qv > bv || (qv == bv && qj < bj)) {
          bv = qv;
          bj = qj;
        }
      }
      // (2) the winner publishes its W row, score and squared norm; every wave fetches the
      // winning row itself through the scalar cache
      // bj names an eligible pool row whenever the block has one; the clamp keeps the row
      // address inside the dictionary whatever the pool holds
      int jstar = __builtin_amdgcn_readfirstlane(bj);
      jstar = jstar < 0 ? 0 : (jstar >= N ? N - 1 : jstar);
      if (elig && j == bj) {
        chosen = true;
        s_sig[k] = sig;
#pragma unroll
        for (int m = 0; m < k; ++m) s_l[buf][m] = W[m];
        s_gdiag[k] = gself;
      }
      if (tid == 0) s_sel[k] = jstar;
      __syncthreads();
      if (gm) {
        float nl2 = 0.f, ly = 0.f;
#pragma unroll
        for (int m = 0; m < k; ++m) {
          const float l = s_l[buf][m];
          nl2 = fmaf(l, l, nl2);
          ly = fmaf(l, s_y[m], ly);
        }
        const float alpha = fmaf(s_gdiag[k], 1.f + ridge_rel, ridge_abs);
        const float Lkk = sqrtf(fmaxf(alpha - nl2, 1e-30f));
        const float yk = (s_sig[k] - ly) / Lkk;
        if (k + 1 < s) {
          const uint32_t *row = reinterpret_cast<const uint32_t *>(dict_atoms + (size_t)jstar * ROWB);
          float acc = row_dot_uniform<DT, NW>(w, row);
#pragma unroll
          for (int m = 0; m < k; ++m) acc = fmaf(-W[m], s_l[buf][m], acc);
          W[k] = acc / Lkk;
          rho = fmaf(-W[k], yk, rho);
        }
        if (tid == 0) {
#pragma unroll
          for (int m = 0; m < k; ++m) s_L[k * SMAX + m] = s_l[buf][m];
          s_L[k * SMAX + k] = Lkk;
          s_y[k] = yk;
        }
      }
    }
  }
  __syncthreads();
  // the chosen rows, for PL's Gram matrix and the residual
  for (int e = tid; e < s * (NW / 4); e += blockDim.x) {
    const int k = e / (NW / 4), c = e % (NW / 4);
    reinterpret_cast<uint4 *>(s_selrow[k])[c] =
        reinterpret_cast<const uint4 *>(dict_atoms + (size_t)s_sel[k] * ROWB)[c];
  }
  __syncthreads();

  if (gm) {
    if (tid == 0) {   // c = L^{-T} y
      for (int i = s - 1; i >= 0; --i) {
        float acc = s_y[i];
        for (int m = i + 1; m < s; ++m) acc = fmaf(-s_L[m * SMAX + i], s_c[m], acc);
        s_c[i] = acc / s_L[i * SMAX + i];
      }
    }
  } else {
    // PL: G_SS from the chosen rows, then Cholesky and two triangular solves on thread 0
    for (int e = tid; e < s * s; e += blockDim.x) {
      const int r = e / s, c = e % s;
      if (c > r) continue;
      float acc = 0.f;
      for (int q = 0; q < NW; ++q) {
        const uint32_t a = s_selrow[r][q], b = s_selrow[c][q];
        if constexpr (DT == DT_F32) acc = fmaf(__uint_as_float(a), __uint_as_float(b), acc);
        else acc = dot2<DT>(a, b, acc);
      }
      s_L[r * SMAX + c] = acc;   // lower triangle of G_SS, factored in place below
    }
    __syncthreads();
    if (tid == 0) {
      for (int r = 0; r < s; ++r) s_L[r * SMAX + r] = fmaf(s_L[r * SMAX + r], 1.f + ridge_rel, ridge_abs);
      for (int c = 0; c < s; ++c) {
        float dcc = s_L[c * SMAX + c];
        for (int m = 0; m < c; ++m) dcc = fmaf(-s_L[c * SMAX + m], s_L[c * SMAX + m], dcc);
        const float Lcc = sqrtf(fmaxf(dcc, 1e-30f));
        s_L[c * SMAX + c] = Lcc;
        for (int r = c + 1; r < s; ++r) {
          float v = s_L[r * SMAX + c];
          for (int m = 0; m < c; ++m) v = fmaf(-s_L[r * SMAX + m], s_L[c * SMAX + m], v);
          s_L[r * SMAX + c] = v / Lcc;
        }
      }
      for (int i = 0; i < s; ++i) {
        float acc = s_sig[i];
        for (int m = 0; m < i; ++m) acc = fmaf(-s_L[i * SMAX + m], s_y[m], acc);
        s_y[i] = acc / s_L[i * SMAX + i];
      }
      for (int i = s - 1; i >= 0; --i) {
        float acc = s_y[i];
        for (int m = i + 1; m < s; ++m) acc = fmaf(-s_L[m * SMAX + i], s_c[m], acc);
        s_c[i] = acc / s_L[i * SMAX + i];
      }
    }
  }
  __syncthreads();

  // residual r = x - D_S^T c from the chosen rows
  float rr = 0.f, xx = 0.f;
  for (int i = tid; i < D; i += blockDim.x) {
    float r = s_x[i];
    for (int k = 0; k < s; ++k) r = fmaf(-s_c[k], lds_elem<DT>(s_selrow[k], i), r);
    rr = fmaf(r, r, rr);
    xx = fmaf(s_x[i], s_x[i], xx);
  }
  rr = wave_sum(rr);
  xx = wave_sum(xx);
  if (lane == 0) {
    s_sum[0][wave] = rr;
    s_sum[1][wave] = xx;
  }
  __syncthreads();
  if (tid < s) {
    out_idx[gv * s + tid] = s_sel[tid];
    out_coef[gv * s + tid] = s_c[tid];
  }
  if (tid == 0) {
    float R = 0.f, Xn = 0.f;
    for (int q = 0; q < nwaves; ++q) {
      R += s_sum[0][q];
      Xn += s_sum[1][q];
    }
    const float e = sqrtf(R / Xn);
    out_relerr[gv] = e;
    out_flags[gv] = e > delta ? FLAG_TRIGGER : 0;
  }
}

#define FADKV_SEL_INST(DT, D, SM)                                                                 \
  template __global__ void select_kernel<DT, D, SM>(                                             \
      const uint8_t *, const uint8_t *, int, int, int, int, int, int, float, float, float, float, \
      const uint16_t *, const float *, const uint8_t *, int32_t *, float *, float *, uint8_t *);
#define FADKV_SEL_INST_D(DT, D) FADKV_SEL_INST(DT, D, 8) FADKV_SEL_INST(DT, D, 16) FADKV_SEL_INST(DT, D, 32)
FADKV_SEL_INST_D(DT_F32, 64)
FADKV_SEL_INST_D(DT_F32, 128)
FADKV_SEL_INST_D(DT_F16, 64)
FADKV_SEL_INST_D(DT_F16, 128)
FADKV_SEL_INST_D(DT_BF16, 64)
FADKV_SEL_INST_D(DT_BF16, 128)

hipError_t launch_select(int dtype, int d, const void *atoms, const void *X, int num_dicts, int N,
                         int M, int n, int s, int select, float ridge_abs, float ridge_rel,
                         float delta_key, float delta_value, const uint16_t *pool_idx,
                         const float *pool_sig, const uint8_t *vstat, int32_t *idx, float *coef,
                         float *relerr, uint8_t *flags, hipStream_t stream) {
  const size_t G = (size_t)num_dicts * M;
  dim3 grid((unsigned)G), block((unsigned)(((n + 63) / 64) * 64));
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
#define L(DT, D, SM)                                                                              \
  hipLaunchKernelGGL((select_kernel<DT, D, SM>), grid, block, 0, stream, A, Xb, num_dicts, N, M, n, s, select, \
                     ridge_abs, ridge_rel, delta_key, delta_value, pool_idx, pool_sig, vstat, idx, \
                     coef, relerr, flags)
#define LS(DT, D) \
  do { if (s <= 8) L(DT, D, 8); else if (s <= 16) L(DT, D, 16); else L(DT, D, 32); } while (0)
#define LD(DT) do { if (d == 64) LS(DT, 64); else LS(DT, 128); } while (0)
  if (dtype == DT_F32) LD(DT_F32);
  else if (dtype == DT_F16) LD(DT_F16);
  else LD(DT_BF16);
#undef LD
#undef LS
#undef L
  return hipGetLastError();
}

}  // namespace fadkv
