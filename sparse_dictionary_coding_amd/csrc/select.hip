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
// Finally r = x - D_S^T c is formed from the chosen rows and e = ||r|| / ||x||.  (PL, which
// needs no pool rows, has its own one-wave kernel in select_pl.hip.)
//
// One workgroup barrier per step.  Before it, every wave reduces its own argmax (DPP) and its
// candidate lane publishes a 64-bit key (|rho| bits, 0xFFFF - atom, wave) together with its
// W row, score and squared norm.  After it, every wave takes the largest key, which names the
// winning atom and the wave whose slot holds the winner's data; the winning row itself is
// read by every wave through the scalar cache.  The slots are double-buffered by step parity:
// a slot written at step k + 2 is written after the barrier of step k + 1, which every reader
// of step k has passed.  After the last step a single wave forms c and the residual.
#include "common.h"
#include "kernels.h"

namespace fadkv {

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
  // the row arrives in chunks of up to 32 words, each chunk's loads issued together, so a
  // step waits on NW / 32 scalar round trips rather than one per 16 words
  constexpr int CHUNK = NW < 32 ? NW : 32;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int h = 0; h < NW; h += CHUNK) {
    uint32_t r[CHUNK];
#pragma unroll
    for (int q = 0; q < CHUNK; ++q) r[q] = row[h + q];
#pragma unroll
    for (int q = 0; q < CHUNK; q += 2) {
      if constexpr (DT == DT_F32) {
        s0 = fmaf(__uint_as_float(a[h + q]), __uint_as_float(r[q]), s0);
        s1 = fmaf(__uint_as_float(a[h + q + 1]), __uint_as_float(r[q + 1]), s1);
      } else {
        s0 = dot2<DT>(a[h + q], r[q], s0);
        s1 = dot2<DT>(a[h + q + 1], r[q + 1], s1);
      }
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

// 16-bit rows with s <= 16 fit 128 VGPRs: 4 waves per SIMD, two 8-wave workgroups per CU.
template <int DT, int D, int SMAX, int MAXW>
__global__ __launch_bounds__(MAXW * 64, (DT != DT_F32 && SMAX <= 16) ? 4 : 1) void select_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int num_dicts, int N, int M,
    int n, int s, float ridge_abs, float ridge_rel, float delta_key, float delta_value,
    const uint16_t *__restrict__ pool_idx, const float *__restrict__ pool_sig,
    const uint8_t *__restrict__ vstat, int32_t *__restrict__ out_idx, float *__restrict__ out_coef,
    float *__restrict__ out_relerr, uint8_t *__restrict__ out_flags, unsigned base) {
  constexpr int NW = RowWords<DT, D>::NW;
  constexpr int ROWB = RowWords<DT, D>::ROWB;
  constexpr int PUB = SMAX + 2;   // published slot: W row, score, squared norm
  __shared__ __attribute__((aligned(16))) uint32_t s_selrow[SMAX][NW];  // chosen rows
  __shared__ float s_L[SMAX * SMAX];   // row k: l of step k (strictly lower part of L)
  __shared__ float s_linv[SMAX], s_y[SMAX];
  __shared__ int s_sel[SMAX];
  __shared__ unsigned long long s_key[2][MAXW];
  __shared__ float s_pub[2][MAXW][PUB];

  // With a multiple of 8 dictionaries, workgroup i (dispatched to XCD i % 8) takes a vector of
  // dictionary xcd + 8 * (r / M), r = i / 8: each dictionary's pool rows are gathered through
  // one XCD's L2.
  // (32-bit arithmetic: num_dicts * M < 2^31 workgroups over all chunks; base is a multiple of
  // 8, so the XCD of workgroup bid is still bid % 8)
  const unsigned bid = base + blockIdx.x, uM = (unsigned)M;
  unsigned dict_u, vec_u;
  if ((num_dicts & 7) == 0) {
    const unsigned r = bid / 8u;
    dict_u = bid % 8u + 8u * (r / uM);
    vec_u = r % uM;
  } else {
    dict_u = bid / uM;
    vec_u = bid % uM;
  }
  const int dict = __builtin_amdgcn_readfirstlane((int)dict_u);
  const size_t gv = (size_t)dict * M + __builtin_amdgcn_readfirstlane(vec_u);
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
  // key slots of absent waves read as "no candidate" (no present wave writes them)
  if (tid < 2 * MAXW && tid % MAXW >= nwaves) s_key[tid / MAXW][tid % MAXW] = 0ull;

  const uint8_t *dict_atoms = atoms + (size_t)dict * N * ROWB;
  const bool act = tid < n;
  int j = 0;
  float sig = 0.f;
  if (act) {
    const int jj = pool_idx[gv * n + tid];
    j = jj < N ? jj : N - 1;   // the screening kernel writes indices < N; never read past the set
    sig = pool_sig[gv * n + tid];
  }
  // each thread loads its own pool row (all 16-byte loads issued back to back); a thread past
  // the pool loads row 0, which it never offers as a candidate
  uint32_t w[NW];
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(dict_atoms + (size_t)j * ROWB);
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const uint4 v = src[q];
      w[4 * q + 0] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
  }
  const float gself = row_self_dot<DT, NW>(w);   // ||d_j||^2, needed if this row is chosen
  // wave 0 keeps x (elements lane and lane + 64) for the residual
  float x0 = 0.f, x1 = 0.f;
  if (wave == 0) {
    const uint8_t *xr = X + gv * ROWB;
    if (lane < D) x0 = elem_f<DT>(xr, lane);
    if (D > 64) x1 = elem_f<DT>(xr, lane + 64);
  }

  float rho = sig;
  float W[SMAX], Y[SMAX];   // Y: y, the same in every lane
#pragma unroll
  for (int m = 0; m < SMAX; ++m) W[m] = Y[m] = 0.f;
  bool chosen = false;

#pragma unroll
  for (int k = 0; k < SMAX; ++k) {
    if (k < s) {
      const int buf = k & 1;
      // wave argmax of |rho| over unchosen entries, ties to the lowest atom index
      const bool elig = act && !chosen;
      float v = elig ? fabsf(rho) : -1.f;
      v = v != v ? 0.f : v;   // a NaN score (non-finite atoms) ranks as 0, never above real ones
      const int wmax = wave_max_nonneg_bits(__float_as_int(v));
      const bool top = elig && __float_as_int(v) == wmax;
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(top);
      int cl = hit ? (int)__ffsll((long long)hit) - 1 : 0;
      if (__popcll(hit) > 1) {
        const int wj = wave_min_i32(top ? j : 0x7fffffff);
        cl = (int)__ffsll((long long)__builtin_amdgcn_ballot_w64(top && j == wj)) - 1;
      }
      const int jc = __builtin_amdgcn_readlane(j, cl);
      const unsigned long long key =
          hit ? ((unsigned long long)(unsigned)wmax << 32) | ((unsigned)(0xFFFF - jc) << 8) |
                    (unsigned)wave
              : 0ull;
      if (lane == cl) {
        s_key[buf][wave] = key;
#pragma unroll
        for (int m = 0; m < k; ++m) s_pub[buf][wave][m] = W[m];
        s_pub[buf][wave][SMAX] = sig;
        s_pub[buf][wave][SMAX + 1] = gself;
      }
      __syncthreads();
      unsigned long long best = s_key[buf][0];
#pragma unroll
      for (int q = 1; q < MAXW; ++q) {
        const unsigned long long kq = s_key[buf][q];
        best = kq > best ? kq : best;
      }
      const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)best);
      const int bw = (int)(lo & (MAXW - 1));
      // a key names an eligible pool row whenever the block has one; the clamp keeps the row
      // address inside the dictionary whatever the pool holds
      int jstar = 0xFFFF - (int)((lo >> 8) & 0xFFFFu);
      jstar = jstar >= N ? N - 1 : jstar;
      const bool win = elig && j == jstar;
      chosen = chosen || win;
      float l[SMAX];
#pragma unroll
      for (int m = 0; m < k; ++m) l[m] = s_pub[buf][bw][m];
      const float sigk = s_pub[buf][bw][SMAX];
      const float gk = s_pub[buf][bw][SMAX + 1];
      // G_{j,j*} for this thread's row: the winning row comes through the scalar cache while
      // the published slot is read
      float acc = 0.f;
      if (k + 1 < s)
        acc = row_dot_uniform<DT, NW>(w, reinterpret_cast<const uint32_t *>(dict_atoms + (size_t)jstar * ROWB));
      if (win) {
#pragma unroll
        for (int q = 0; q < NW / 4; ++q)
          reinterpret_cast<uint4 *>(s_selrow[k])[q] =
              make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
      }
      {
        float nl2 = 0.f, ly = 0.f;
#pragma unroll
        for (int m = 0; m < k; ++m) {
          nl2 = fmaf(l[m], l[m], nl2);
          ly = fmaf(l[m], Y[m], ly);
        }
        const float alpha = fmaf(gk, 1.f + ridge_rel, ridge_abs);
        const float invL = __builtin_amdgcn_rsqf(fmaxf(alpha - nl2, 1e-30f));
        // y is the same in every lane: keep it in scalar registers
        const float yk = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int((sigk - ly) * invL)));
        Y[k] = yk;
        if (k + 1 < s) {
#pragma unroll
          for (int m = 0; m < k; ++m) acc = fmaf(-W[m], l[m], acc);
          W[k] = acc * invL;
          rho = fmaf(-W[k], yk, rho);
        }
        if (tid == 0) {
#pragma unroll
          for (int m = 0; m < k; ++m) s_L[k * SMAX + m] = l[m];
          s_linv[k] = invL;
          s_y[k] = yk;
        }
      }
      if (tid == 0) s_sel[k] = jstar;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // ---- one wave: coefficients, residual, outputs ----
  float c = 0.f;   // lane k < s holds c_k
  {
    // c = L^{-T} y: lane m carries t_m = y_m - sum_{i > m} L_im c_i; column i is finished
    // once every later column has been folded in, so c_i = t_i / L_ii is final at step i
    float t = lane < s ? s_y[lane < SMAX ? lane : 0] : 0.f;
    float lcol[SMAX];
#pragma unroll
    for (int i = 0; i < SMAX; ++i) lcol[i] = (i < s && lane < i) ? s_L[i * SMAX + lane] : 0.f;
#pragma unroll
    for (int i = SMAX - 1; i >= 0; --i) {
      if (i < s) {
        const float ci = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), i)) * s_linv[i];
        t = fmaf(-lcol[i], ci, t);
      }
    }
    c = lane < s ? t * s_linv[lane < SMAX ? lane : 0] : 0.f;
  }

  // residual r = x - D_S^T c from the chosen rows; lane i holds elements i and i + 64
  float r0 = x0, r1 = x1;
#pragma unroll
  for (int k = 0; k < SMAX; ++k) {
    if (k < s) {
      const float ck = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), k));
      if (lane < D) r0 = fmaf(-ck, lds_elem<DT>(s_selrow[k], lane), r0);
      if (D > 64) r1 = fmaf(-ck, lds_elem<DT>(s_selrow[k], lane + 64), r1);
    }
  }
  const float rr = wave_sum(fmaf(r0, r0, r1 * r1));
  const float xx = wave_sum(fmaf(x0, x0, x1 * x1));
  if (lane < s) {
    out_idx[gv * s + lane] = s_sel[lane < SMAX ? lane : 0];
    out_coef[gv * s + lane] = c;
  }
  if (lane == 0) {
    const float e = sqrtf(rr / xx);
    out_relerr[gv] = e;
    out_flags[gv] = e > delta ? FLAG_TRIGGER : 0;
  }
}

#define FADKV_SEL_INST(DT, D, SM, MW)                                                             \
  template __global__ void select_kernel<DT, D, SM, MW>(                                         \
      const uint8_t *, const uint8_t *, int, int, int, int, int, float, float, float, float,      \
      const uint16_t *, const float *, const uint8_t *, int32_t *, float *, float *, uint8_t *,  \
      unsigned);
#define FADKV_SEL_INST_S(DT, D, SM) FADKV_SEL_INST(DT, D, SM, 4) FADKV_SEL_INST(DT, D, SM, 8)
#define FADKV_SEL_INST_D(DT, D) \
  FADKV_SEL_INST_S(DT, D, 8) FADKV_SEL_INST_S(DT, D, 16) FADKV_SEL_INST_S(DT, D, 32)
FADKV_SEL_INST_D(DT_F32, 64)
FADKV_SEL_INST_D(DT_F32, 128)
FADKV_SEL_INST_D(DT_F16, 64)
FADKV_SEL_INST_D(DT_F16, 128)
FADKV_SEL_INST_D(DT_BF16, 64)
FADKV_SEL_INST_D(DT_BF16, 128)

hipError_t launch_select(int dtype, int d, const void *atoms, const void *X, int num_dicts, int N,
                         int M, int n, int s, float ridge_abs, float ridge_rel,
                         float delta_key, float delta_value, const uint16_t *pool_idx,
                         const float *pool_sig, const uint8_t *vstat, int32_t *idx, float *coef,
                         float *relerr, uint8_t *flags, hipStream_t stream) {
  const size_t G = (size_t)num_dicts * M;
  const unsigned threads = (unsigned)(((n + 63) / 64) * 64);   // n <= 512: at most 8 waves
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
  for (size_t b0 = 0; b0 < G; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = G - b0 < kMaxBlocksPerLaunch ? G - b0 : kMaxBlocksPerLaunch;
    const dim3 grid((unsigned)nb), block(threads);
#define L(DT, D, SM, MW)                                                                          \
  hipLaunchKernelGGL((select_kernel<DT, D, SM, MW>), grid, block, 0, stream, A, Xb, num_dicts, N, \
                     M, n, s, ridge_abs, ridge_rel, delta_key, delta_value, pool_idx,              \
                     pool_sig, vstat, idx, coef, relerr, flags, (unsigned)b0)
#define LW(DT, D, SM) do { if (threads <= 256) L(DT, D, SM, 4); else L(DT, D, SM, 8); } while (0)
#define LS(DT, D) \
  do { if (s <= 8) LW(DT, D, 8); else if (s <= 16) LW(DT, D, 16); else LW(DT, D, 32); } while (0)
#define LD(DT) do { if (d == 64) LS(DT, 64); else LS(DT, 128); } while (0)
    if (dtype == DT_F32) LD(DT_F32);
    else if (dtype == DT_F16) LD(DT_F16);
    else LD(DT_BF16);
#undef LD
#undef LS
#undef LW
#undef L
  }
  return hipGetLastError();
}

}  // namespace fadkv
