// Full-dictionary greedy yardstick: the "full-OMP atoms" of FAD-KV Figure 1b and the Cost 1.00
// row of Table 4.  It takes the same greedy steps as the GM selection (largest |rho_j|, ties to
// the lowest index, the Table 5 ridge system re-solved at every step) with every atom of the
// dictionary a candidate instead of the Top-n pool, so it measures what the screening saves.
//
// Step k (k = 0 .. s-1) is two launches:
//   omp_corr_kernel   rho_j = <d_j, r> for every atom j and vector on the matrix cores (16-atom
//                     dictionary tiles through LDS, as in the screening kernel), then per vector
//                     the largest |rho_j| over atoms not yet chosen.  The residual r is fp32;
//                     the MFMA takes it as a sum of parts in the storage dtype (f16: two parts of
//                     11 significant bits, bf16: three of 8, after scaling r by a power of two
//                     so that the parts stay normal), so every product is exact and the sum is
//                     accumulated in fp32.  At k = 0, r = x itself (one part, read from X).
//   omp_update_kernel one wave per vector: appends the chosen atom, extends the Cholesky factor
//                     of G_SS + diag(ridge_abs + ridge_rel G_jj) by one row, solves for c,
//                     forms r = x - D_S^T c in fp32 and stores its parts; the last step writes
//                     the code (atoms in selection order, c, relative error, trigger flag).
// omp_init_kernel runs first: zero and non-finite vectors get the empty code (relative error
// 0, or NaN with flag NONFINITE) and the steps skip them.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace fadkv {

namespace {

using namespace tile;

constexpr int CVT = 32;            // vectors per correlation workgroup (two MFMA blocks)
constexpr int CWAVES = 8;
constexpr int CTHREADS = CWAVES * 64;
constexpr int SMAXALL = 32;        // largest sparsity the library accepts
constexpr int SENTINEL = 0x7fffffff;

typedef unsigned long long u64;

template <int DT> struct Parts;
template <> struct Parts<DT_F32> { static constexpr int n = 1; };
template <> struct Parts<DT_F16> { static constexpr int n = 2; };
template <> struct Parts<DT_BF16> { static constexpr int n = 3; };

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((u64)hi << 32) | lo;
}

// storage-dtype element from a float (round to nearest even), as its bits
template <int DT> __device__ __forceinline__ uint32_t to_bits(float f) {
  if constexpr (DT == DT_F16) return float_to_f16_bits(f);
  else return float_to_bf16_bits(f);
}
template <int DT> __device__ __forceinline__ float from_bits(uint32_t b) {
  if constexpr (DT == DT_F16) return f16_bits_to_float(b);
  else return bf16_bits_to_float(b);
}

// <a, b> of two stored rows by one lane (fp32 accumulation)
template <int DT, int D>
__device__ __forceinline__ float lane_row_dot(const uint8_t *a, const uint8_t *b) {
  constexpr int CPR = D * Elem<DT>::bytes / 16;
  const uint4 *pa = reinterpret_cast<const uint4 *>(a);
  const uint4 *pb = reinterpret_cast<const uint4 *>(b);
  float acc = 0.f;
#pragma unroll 4
  for (int c = 0; c < CPR; ++c) {
    const uint4 u = pa[c], v = pb[c];
    if constexpr (DT == DT_F32) {
      acc = fmaf(__uint_as_float(u.x), __uint_as_float(v.x), acc);
      acc = fmaf(__uint_as_float(u.y), __uint_as_float(v.y), acc);
      acc = fmaf(__uint_as_float(u.z), __uint_as_float(v.z), acc);
      acc = fmaf(__uint_as_float(u.w), __uint_as_float(v.w), acc);
    } else {
      acc = dot2<DT>(u.x, v.x, acc);
      acc = dot2<DT>(u.y, v.y, acc);
      acc = dot2<DT>(u.z, v.z, acc);
      acc = dot2<DT>(u.w, v.w, acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace

// ---- classification ------------------------------------------------------------------------

template <int DT, int D>
__global__ __launch_bounds__(256) void omp_init_kernel(const uint8_t *__restrict__ X, size_t G,
                                                       int s, uint8_t *__restrict__ status,
                                                       int32_t *__restrict__ idx,
                                                       float *__restrict__ coef,
                                                       float *__restrict__ relerr,
                                                       uint8_t *__restrict__ flags, size_t base) {
  constexpr int ROWB = D * Elem<DT>::bytes;
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const size_t gv = base + (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gv >= G) return;
  const uint8_t *xr = X + gv * ROWB;
  float ss = 0.f;
  bool fin = true;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const float v = elem_f<DT>(xr, lane + 64 * p);
    fin = fin && __builtin_isfinite(v);
    ss = fmaf(v, v, ss);
  }
  const bool all_fin = __builtin_amdgcn_ballot_w64(!fin) == 0;
  ss = wave_sum_f(ss);
  const uint8_t st = !all_fin ? VS_NONFINITE : (ss == 0.f ? VS_ZERO : VS_NORMAL);
  if (lane == 0) status[gv] = st;
  if (st != VS_NORMAL) {
    if (lane < s) {
      idx[gv * s + lane] = -1;
      coef[gv * s + lane] = 0.f;
    }
    if (lane == 0) {
      relerr[gv] = st == VS_NONFINITE ? __builtin_nanf("") : 0.f;
      flags[gv] = st == VS_NONFINITE ? FLAG_NONFINITE : 0;
    }
  }
}

// ---- correlation sweep + argmax ------------------------------------------------------------

// R: rparts rows per vector (row p of vector g at R + (g * rparts + p) * ROWB), of which the
// first nparts are summed.  S: [G][s] atoms chosen so far (first k valid).
template <int DT, int D>
__global__ __launch_bounds__(CTHREADS) void omp_corr_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ R, int rparts, int nparts,
    int num_dicts, int N, int M, const int32_t *__restrict__ S, int s, int k,
    int32_t *__restrict__ jstar) {
  using G = Geo<DT, D>;
  constexpr int NP = Parts<DT>::n;
  __shared__ __attribute__((aligned(16))) uint4 s_stage[CWAVES * G::STAGE];
  __shared__ int s_sorted[CVT][SMAXALL + 1];
  __shared__ u64 s_best[CWAVES][CVT];

  // same workgroup -> (dictionary, vector block) numbering as the screening kernel
  const int nvb = (M + CVT - 1) / CVT;
  const int xcd = blockIdx.x % 8, rr = blockIdx.x / 8;
  const int dict = xcd + 8 * (rr / nvb);
  if (dict >= num_dicts) return;
  const int v0 = (rr % nvb) * CVT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t *dict_atoms = atoms + (size_t)dict * N * G::ROWB;
  const size_t vbase = (size_t)dict * M + v0;
  uint4 *stage = s_stage + wave * G::STAGE;
  const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)stage);

  if (tid < CVT) {
    // the vector's chosen atoms, ascending, then a sentinel
    int *srt = s_sorted[tid];
    const int cnt = v0 + tid < M ? k : 0;
    for (int i = 0; i < cnt; ++i) {
      const int a = S[(vbase + tid) * s + i];
      int j = i;
      while (j > 0 && srt[j - 1] > a) {
        srt[j] = srt[j - 1];
        --j;
      }
      srt[j] = a;
    }
    srt[cnt] = SENTINEL;
  }
  // B fragments of every residual part: block b, step i = chunk 4 i + lane / 16 of vector
  // 16 b + lane % 16
  uint4 bf[NP][2][G::CH];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int v = 16 * b + lane % 16;
      const bool ok = p < nparts && v0 + v < M;
      const uint4 *src = reinterpret_cast<const uint4 *>(
          R + ((vbase + (ok ? v : 0)) * rparts + (ok ? p : 0)) * G::ROWB);
#pragma unroll
      for (int i = 0; i < G::CH; ++i) bf[p][b][i] = ok ? src[4 * i + lane / 16] : make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();

  const int r = lane % 16, g = lane / 16;
  const int ntiles = (N + 15) / 16;
  u64 best[2] = {0ull, 0ull};
  int ptr[2] = {0, 0}, nx[2];
  nx[0] = s_sorted[r][0];
  nx[1] = s_sorted[16 + r][0];
  if (wave < ntiles) {
    uint32_t off[G::LOADS];
    tile_offsets<DT, D>(lane, off);
    issue_tile<DT, D>(dict_atoms, N, wave, lane, off, stage_lds);
    for (int t = wave; t < ntiles; t += CWAVES) {
      wait_vmem();
      uint4 a[G::CH];
#pragma unroll
      for (int i = 0; i < G::CH; ++i) a[i] = stage[r * G::CPR + ((4 * i + g) ^ swz<G::CPR>(r))];
      wait_lds();
      if (t + CWAVES < ntiles) issue_tile<DT, D>(dict_atoms, N, t + CWAVES, lane, off, stage_lds);
      float4_t acc[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (p < nparts) tile_mma<DT, D>(a, bf[p], acc[0], acc[1]);
      const int atom0 = t * 16 + 4 * g;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // chosen atoms among this lane's four: advance through the sorted list (atoms below
        // atom0 belong to other lanes' groups or earlier tiles)
        uint32_t ex = 0;
        while (nx[b] < atom0 + 4) {
          if (nx[b] >= atom0) ex |= 1u << (nx[b] - atom0);
          nx[b] = s_sorted[16 * b + r][++ptr[b]];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int atom = atom0 + e;
          const u64 key = ((u64)(__float_as_uint(acc[b][e]) & 0x7fffffffu) << 16) |
                          (u64)(0xFFFFu - (uint32_t)atom);
          const bool ok = atom < N && !((ex >> e) & 1u);
          best[b] = ok && key > best[b] ? key : best[b];
        }
      }
    }
  }
  // lanes r, r + 16, r + 32, r + 48 hold the same vectors
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    u64 o = shfl_xor_u64(best[b], 16);
    best[b] = o > best[b] ? o : best[b];
    o = shfl_xor_u64(best[b], 32);
    best[b] = o > best[b] ? o : best[b];
  }
  if (lane < 16) {
    s_best[wave][lane] = best[0];
    s_best[wave][16 + lane] = best[1];
  }
  __syncthreads();
  if (tid < CVT && v0 + tid < M) {
    u64 b = 0;
#pragma unroll
    for (int w = 0; w < CWAVES; ++w) b = s_best[w][tid] > b ? s_best[w][tid] : b;
    jstar[vbase + tid] = b == 0 ? -1 : (int)(0xFFFFu - (uint32_t)(b & 0xFFFFu));
  }
}

// ---- one greedy step per vector ------------------------------------------------------------

// Lm: [G][s][s] Cholesky rows (row i holds L[i][0..i]); sig: [G][s] <d_S[i], x>.
template <int DT, int D, int SMAX>
__global__ __launch_bounds__(256) void omp_update_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int N, int M, size_t G,
    int s, int k, float ridge_abs, float ridge_rel, float delta_key, float delta_value,
    uint8_t *__restrict__ status, const int32_t *__restrict__ jstar,
    int32_t *__restrict__ S, float *__restrict__ Lm, float *__restrict__ sig,
    uint8_t *__restrict__ R, int32_t *__restrict__ idx, float *__restrict__ coef,
    float *__restrict__ relerr, uint8_t *__restrict__ flags, size_t base) {
  constexpr int ROWB = D * Elem<DT>::bytes;
  constexpr int PER = D / 64;
  constexpr int NP = Parts<DT>::n;
  const int lane = threadIdx.x & 63;
  const size_t gv = base + (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gv >= G) return;
  if (status[gv] != VS_NORMAL) return;
  const int dict = (int)(gv / (size_t)M);
  const uint8_t *dict_atoms = atoms + (size_t)dict * N * ROWB;
  const uint8_t *xr = X + gv * ROWB;
  const int j = jstar[gv];
  if (j < 0 || j >= N) {
    // no candidate (cannot happen with s <= N, which the host checks): give the vector the
    // non-finite code and take it out of the remaining steps
    if (lane < s) {
      idx[gv * s + lane] = -1;
      coef[gv * s + lane] = 0.f;
    }
    if (lane == 0) {
      relerr[gv] = __builtin_nanf("");
      flags[gv] = FLAG_NONFINITE;
      status[gv] = VS_NONFINITE;
    }
    return;
  }
  const uint8_t *dj = dict_atoms + (size_t)j * ROWB;
  int32_t *Sg = S + gv * s;
  float *Lg = Lm + gv * (size_t)s * s;
  float *sg = sig + gv * s;

  // lane i < k: chosen atom i, its Cholesky row (strictly lower part and diagonal) and
  // <d_i, x>; lane k: the new atom
  const int si = lane < k ? Sg[lane] : (lane == k ? j : -1);
  float Lrow[SMAX], Lcol[SMAX];
  float dg = 0.f, b = 0.f;
#pragma unroll
  for (int m = 0; m < SMAX; ++m) {
    Lrow[m] = (m < lane && lane < k) ? Lg[lane * s + m] : 0.f;   // L[lane][m]
    Lcol[m] = (lane < m && m < k) ? Lg[m * s + lane] : 0.f;      // L[m][lane]
  }
  if (lane < k) {
    dg = Lg[lane * s + lane];
    b = sg[lane];
  }
  // lane i < k: <d_j, d_S[i]>; lane k: <d_j, d_j>; lane k + 1: <d_j, x>
  float dv = 0.f;
  if (lane <= k + 1) {
    const uint8_t *row = lane < k ? dict_atoms + (size_t)si * ROWB : (lane == k ? dj : xr);
    dv = lane_row_dot<DT, D>(dj, row);
  }
  const float gjj = __shfl(dv, k);
  const float sj = __shfl(dv, k + 1);

  // new Cholesky row: L[k][m] = (g_m - sum_{l<m} L[k][l] L[m][l]) / L[m][m]
  float gcol = lane < k ? dv : 0.f;
  float mine = 0.f, sumsq = 0.f;
#pragma unroll
  for (int m = 0; m < SMAX; ++m) {
    if (m < k) {
      const float lm = __shfl(gcol, m) / __shfl(dg, m);
      sumsq = fmaf(lm, lm, sumsq);
      if (lane == m) mine = lm;
      if (lane == k) Lrow[m] = lm;
      if (lane > m) gcol = fmaf(-Lrow[m], lm, gcol);
    }
  }
  const float lkk = sqrtf(gjj + (ridge_abs + ridge_rel * gjj) - sumsq);
  if (lane < k) Lg[k * s + lane] = mine;
  if (lane == k) {
    Lg[k * s + k] = lkk;
    sg[k] = sj;
    Sg[k] = j;
    dg = lkk;
    b = sj;
  }

  // forward: y = L^{-1} sigma_S
  float y = 0.f;
#pragma unroll
  for (int m = 0; m < SMAX; ++m) {
    if (m <= k) {
      const float ym = __shfl(b, m) / __shfl(dg, m);
      if (lane == m) y = ym;
      if (lane > m) b = fmaf(-Lrow[m], ym, b);
    }
  }
  // backward: c = L^{-T} y (lane i holds c_i)
  float c = 0.f;
#pragma unroll
  for (int m = SMAX - 1; m >= 0; --m) {
    if (m <= k) {
      const float cm = __shfl(y, m) / __shfl(dg, m);
      if (lane == m) c = cm;
      if (lane < m) y = fmaf(-(m == k ? mine : Lcol[m]), cm, y);
    }
  }

  // residual r = x - sum_m c_m d_S[m] in fp32
  float rv[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) rv[p] = elem_f<DT>(xr, lane + 64 * p);
#pragma unroll
  for (int m = 0; m < SMAX; ++m) {
    if (m <= k) {
      const float cm = __shfl(c, m);
      const uint8_t *row = dict_atoms + (size_t)__shfl(si, m) * ROWB;
#pragma unroll
      for (int p = 0; p < PER; ++p) rv[p] = fmaf(-cm, elem_f<DT>(row, lane + 64 * p), rv[p]);
    }
  }

  if (k + 1 < s) {
    uint8_t *Rg = R + gv * NP * ROWB;
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int p = 0; p < PER; ++p) reinterpret_cast<float *>(Rg)[lane + 64 * p] = rv[p];
    } else {
      // scale by a power of two so that max |r| is in [1, 2): the parts stay normal numbers
      float mx = 0.f;
#pragma unroll
      for (int p = 0; p < PER; ++p) mx = fmaxf(mx, fabsf(rv[p]));
      mx = wave_max_f(mx);
      int e = 0;
      if (mx > 0.f) {
        (void)__builtin_frexpf(mx, &e);   // mx = f 2^e, f in [0.5, 1)
        e -= 1;
      }
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        float rest = __builtin_ldexpf(rv[p], -e);
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const uint32_t hb = to_bits<DT>(rest);
          reinterpret_cast<uint16_t *>(Rg + q * ROWB)[lane + 64 * p] = (uint16_t)hb;
          rest -= from_bits<DT>(hb);
        }
      }
    }
    return;
  }

  // last step: the code
  float rr = 0.f, xx = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const float xv = elem_f<DT>(xr, lane + 64 * p);
    rr = fmaf(rv[p], rv[p], rr);
    xx = fmaf(xv, xv, xx);
  }
  rr = wave_sum_f(rr);
  xx = wave_sum_f(xx);
  const float e = sqrtf(rr) / sqrtf(xx);
  if (lane < s) {
    idx[gv * s + lane] = si;
    coef[gv * s + lane] = c;
  }
  if (lane == 0) {
    relerr[gv] = e;
    flags[gv] = e > ((dict & 1) ? delta_value : delta_key) ? FLAG_TRIGGER : 0;
  }
}

// ---- host ----------------------------------------------------------------------------------

namespace {

template <int DT, int D, int SMAX>
void launch_update(const OmpArgs &a, int k, hipStream_t stream) {
  const size_t G = (size_t)a.num_dicts * a.M;
  const size_t blocks = (G + 3) / 4;
  for (size_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
    hipLaunchKernelGGL((omp_update_kernel<DT, D, SMAX>), dim3((unsigned)nb), dim3(256), 0,
                       stream, static_cast<const uint8_t *>(a.atoms),
                       static_cast<const uint8_t *>(a.X), a.N, a.M, G, a.s, k, a.ridge_abs,
                       a.ridge_rel, a.delta_key, a.delta_value, a.status, a.jstar, a.S, a.L,
                       a.sig, a.R, a.idx, a.coef, a.relerr, a.flags, b0 * 4);
  }
}

template <int DT, int D>
hipError_t run(const OmpArgs &a, hipStream_t stream) {
  const size_t G = (size_t)a.num_dicts * a.M;
  const uint8_t *A = static_cast<const uint8_t *>(a.atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(a.X);
  const size_t blocks = (G + 3) / 4;
  for (size_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
    hipLaunchKernelGGL((omp_init_kernel<DT, D>), dim3((unsigned)nb), dim3(256), 0, stream, Xb, G,
                       a.s, a.status, a.idx, a.coef, a.relerr, a.flags, b0 * 4);
  }
  const int nvb = (a.M + CVT - 1) / CVT;
  const dim3 cgrid((unsigned)(8 * ((a.num_dicts + 7) / 8) * nvb));
  for (int k = 0; k < a.s; ++k) {
    const uint8_t *Rin = k == 0 ? Xb : a.R;
    const int rparts = k == 0 ? 1 : Parts<DT>::n;
    hipLaunchKernelGGL((omp_corr_kernel<DT, D>), cgrid, dim3(CTHREADS), 0, stream, A, Rin, rparts,
                       rparts, a.num_dicts, a.N, a.M, a.S, a.s, k, a.jstar);
    if (a.s <= 8) launch_update<DT, D, 8>(a, k, stream);
    else if (a.s <= 16) launch_update<DT, D, 16>(a, k, stream);
    else launch_update<DT, D, 32>(a, k, stream);
  }
  return hipGetLastError();
}

}  // namespace

size_t omp_residual_row_bytes(int dtype, int d) {
  const int parts = dtype == DT_F32 ? 1 : (dtype == DT_F16 ? 2 : 3);
  return (size_t)parts * d * (dtype == DT_F32 ? 4 : 2);
}

hipError_t launch_omp(int dtype, int d, const OmpArgs &a, hipStream_t stream) {
  if (dtype == DT_F32) return d == 64 ? run<DT_F32, 64>(a, stream) : run<DT_F32, 128>(a, stream);
  if (dtype == DT_F16) return d == 64 ? run<DT_F16, 64>(a, stream) : run<DT_F16, 128>(a, stream);
  return d == 64 ? run<DT_BF16, 64>(a, stream) : run<DT_BF16, 128>(a, stream);
}

}  // namespace fadkv
