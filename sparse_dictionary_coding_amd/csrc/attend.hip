// Decode attention over sparse-coded keys and values (the consumer of the encoder's codes).
//
// A cached key is k_t = sum_k cK[t][k] d^K_{iK[t][k]}, so <q, k_t> = sum_k cK[t][k] qd[iK[t][k]]
// with qd = D_K q computed once per query, and sum_t p_t v_t = w . D_V with the softmax weights
// scattered onto the value atoms, w[j] = sum_{t,k: iV[t][k] = j} p_t cV[t][k].  Three kernels:
//   attend_qd       qd[query][j] = <q, d^K_j>: v_mfma_f32_16x16x32 (16x16x4 for fp32), 64 queries
//                   x 128 atoms per workgroup
//   attend_softmax  one workgroup per (row, query group): qd rows in LDS, a max pass and an
//                   exp/sum/scatter pass over the row's tokens (s LDS gathers per token and
//                   query, exact 64-bit fixed-point LDS atomics onto w), then w / sum written
//                   over qd
//   attend_out      part[range][query] = w[query][range] . D_V[range] for 32 queries x 128 atoms
//                   per workgroup (fp32 register tiles over LDS-staged chunks)
//   attend_reduce   out = sum over the ranges of part
#include "common.h"
#include "kernels.h"

namespace fadkv {

namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));

template <int DT, int D> struct AGeo {
  static constexpr int ROWB = D * Elem<DT>::bytes;
  static constexpr int CH = ROWB / 64;   // 16-byte chunks per lane per row (4 i + lane / 16)
};

template <int DT>
__device__ __forceinline__ void mfma_chunk(const uint4 &a, const uint4 &b, float4_t &c) {
  if constexpr (DT == DT_F16) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                               __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  } else if constexpr (DT == DT_BF16) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
}

constexpr int QD_QUERIES = 64;     // four 16-query blocks
constexpr int QD_ATOMS = 128;      // 8 tiles of 16 atoms, two per wave
constexpr int SM_THREADS = 1024;   // 16 waves: four per SIMD hide the code loads
constexpr int SM_GMAX = 8;         // queries per softmax workgroup
constexpr int SM_CH = 8;           // slots loaded together
constexpr int SM_LDS_FLOATS = 32768;   // qd rows + fp32 weights: 128 KB
constexpr int SM_LDS_FIXED = 156 * 1024;   // qd rows + 64-bit fixed-point weights
constexpr int OUT_QUERIES = 32;
constexpr int OUT_ATOMS = 128;

}  // namespace

// qd[query][j] = <q[query], d^K_j>; block b of the workgroup's 64 queries is the B operand
// (column = query), each 16-atom tile the A operand (row = atom); lane l holds chunk
// 4 i + l / 16 of row l % 16 on both sides, so the product sums over all of d.
template <int DT, int D>
__global__ __launch_bounds__(256) void attend_qd_kernel(const uint8_t *__restrict__ dictK,
                                                        const uint8_t *__restrict__ Q, int RG,
                                                        int N, float *__restrict__ qd) {
  using G = AGeo<DT, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q0 = blockIdx.x * QD_QUERIES;
  const int r16 = lane & 15, g4 = lane >> 4;
  uint4 b[4][G::CH];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int qq = q0 + 16 * k + r16;
    const bool ok = qq < RG;
    const uint4 *src = reinterpret_cast<const uint4 *>(Q + (size_t)(ok ? qq : 0) * G::ROWB);
#pragma unroll
    for (int i = 0; i < G::CH; ++i) b[k][i] = ok ? src[4 * i + g4] : make_uint4(0, 0, 0, 0);
  }
  for (int m = 0; m < QD_ATOMS / 16 / 4; ++m) {
    const int t = blockIdx.y * (QD_ATOMS / 16) + wave + 4 * m;
    if (t * 16 >= N) break;
    int row = t * 16 + r16;
    row = row < N ? row : N - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(dictK + (size_t)row * G::ROWB);
    uint4 a[G::CH];
#pragma unroll
    for (int i = 0; i < G::CH; ++i) a[i] = src[4 * i + g4];
    float4_t acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < G::CH; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) mfma_chunk<DT>(a[i], b[k][i], acc[k]);
    }
    // lane l holds query column l % 16 of each block, atoms 4 (l / 16) + e of the tile
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int qq = q0 + 16 * k + r16;
      if (qq >= RG) continue;
      const int j = t * 16 + 4 * g4;
      float *dst = qd + (size_t)qq * N + j;
      if (j + 4 <= N && (N & 3) == 0) {
        *reinterpret_cast<float4_t *>(dst) = acc[k];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < N) dst[e] = acc[k][e];
      }
    }
  }
}

// up to SM_CH slots of a token (rem = slots left); 16-byte loads when every token's slots start
// 16-byte aligned (s a multiple of 4), else 4-byte loads.  Missing slots read as empty.
__device__ __forceinline__ void load_slots(const int32_t *__restrict__ idx,
                                           const float *__restrict__ coef, int rem, bool vec,
                                           int (&j)[SM_CH], float (&c)[SM_CH]) {
  if (vec) {
#pragma unroll
    for (int q = 0; q < SM_CH / 4; ++q) {
      int4 iv = make_int4(-1, -1, -1, -1);
      float4 cv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * q < rem) {
        iv = reinterpret_cast<const int4 *>(idx)[q];
        cv = reinterpret_cast<const float4 *>(coef)[q];
      }
      j[4 * q] = iv.x; j[4 * q + 1] = iv.y; j[4 * q + 2] = iv.z; j[4 * q + 3] = iv.w;
      c[4 * q] = cv.x; c[4 * q + 1] = cv.y; c[4 * q + 2] = cv.z; c[4 * q + 3] = cv.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < SM_CH; ++k) {
      j[k] = k < rem ? idx[k] : -1;
      c[k] = k < rem ? coef[k] : 0.f;
    }
  }
}

// z[g] = sum_k coef[k] qs[g][idx[k]] over the token's valid slots; the slots are loaded SM_CH
// at a time before their gathers, so those loads are in flight together.
__device__ __forceinline__ void logits(const int32_t *__restrict__ idx,
                                       const float *__restrict__ coef, int s, int N, int gn,
                                       const float *qs, float (&z)[SM_GMAX]) {
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) z[g] = 0.f;
  for (int k0 = 0; k0 < s; k0 += SM_CH) {
    int j[SM_CH];
    float c[SM_CH];
    load_slots(idx + k0, coef + k0, s - k0, (s & 3) == 0, j, c);
#pragma unroll
    for (int k = 0; k < SM_CH; ++k) {
      if (j[k] >= 0 && j[k] < N) {
#pragma unroll
        for (int g = 0; g < SM_GMAX; ++g)
          if (g < gn) z[g] = fmaf(c[k], qs[g * N + j[k]], z[g]);
      }
    }
  }
}

// One workgroup per (row, group of up to SM_GMAX queries).
//
// FIXED: the value weights are accumulated as 64-bit integers, each contribution p_t cV[t][k]
// (fp32) scaled by 2^sh and converted exactly; sh is the largest power of two that keeps
// len * max|cV| * 2^sh below 2^61, so the integer sums cannot overflow and are exact (LDS
// integer atomics run several times faster than fp32 ones).  Otherwise fp32 LDS atomics (the
// fallback when the 8-byte accumulators of N atoms do not fit the LDS budget).
template <bool FIXED>
__global__ __launch_bounds__(SM_THREADS) void attend_softmax_kernel(
    const int32_t *__restrict__ k_idx, const float *__restrict__ k_coef,
    const int32_t *__restrict__ v_idx, const float *__restrict__ v_coef,
    const int32_t *__restrict__ lens, int T, int s, int N, int G, int gw, float scale,
    float *__restrict__ ws) {
  // dynamic LDS starts after the static variables: the 16-byte alignment keeps the 64-bit
  // weights below 8-byte aligned whatever the static part adds up to
  extern __shared__ __attribute__((aligned(16))) float s_lds[];
  __shared__ float s_red[SM_THREADS / 64][SM_GMAX];
  __shared__ float s_cred[SM_THREADS / 64];
  __shared__ float s_m[SM_GMAX], s_sum[SM_GMAX];
  __shared__ int s_sh;
  const int r = blockIdx.x;
  const int g0 = blockIdx.y * gw;
  const int gn = min(gw, G - g0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int L = lens[r];
  L = L < 0 ? 0 : (L > T ? T : L);
  float *qs = s_lds;                 // [gn][N] qd rows
  float *wv = s_lds + (size_t)gw * N;   // [gn][N] value-atom weights (fp32)
  // FIXED: [gn][N] 64-bit weights after the qd rows, 8-byte aligned
  unsigned long long *wq =
      reinterpret_cast<unsigned long long *>(s_lds + (((size_t)gw * N + 1) & ~(size_t)1));
  float *rows = ws + ((size_t)r * G + g0) * N;
  for (int i = tid; i < gn * N; i += SM_THREADS) {
    qs[i] = rows[i];
    if constexpr (FIXED) wq[i] = 0ull;
    else wv[i] = 0.f;
  }
  __syncthreads();
  const size_t cbase = (size_t)r * T * s;

  // pass 1: the largest logit of every query (and, FIXED, the largest |cV|)
  float mx[SM_GMAX];
  float cmax = 0.f;
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) mx[g] = -__builtin_inff();
  for (int t = tid; t < L; t += SM_THREADS) {
    float z[SM_GMAX];
    logits(k_idx + cbase + (size_t)t * s, k_coef + cbase + (size_t)t * s, s, N, gn, qs, z);
#pragma unroll
    for (int g = 0; g < SM_GMAX; ++g) mx[g] = fmaxf(mx[g], z[g] * scale);
    if constexpr (FIXED) {
      for (int k = 0; k < s; ++k) {
        const int j = v_idx[cbase + (size_t)t * s + k];
        if (j >= 0 && j < N) cmax = fmaxf(cmax, fabsf(v_coef[cbase + (size_t)t * s + k]));
      }
    }
  }
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) {
    float v = mx[g];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0) s_red[wave][g] = v;
  }
  if constexpr (FIXED) {
    float v = cmax;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0) s_cred[wave] = v;
  }
  __syncthreads();
  if (tid < SM_GMAX) {
    float v = s_red[0][tid];
    for (int w = 1; w < SM_THREADS / 64; ++w) v = fmaxf(v, s_red[w][tid]);
    s_m[tid] = v;
  }
  if (FIXED && tid == 0) {
    float v = 0.f;
    for (int w = 0; w < SM_THREADS / 64; ++w) v = fmaxf(v, s_cred[w]);
    // len * cmax * 2^sh < 2^61: with len * cmax in [2^(e-1), 2^e), sh = 61 - e
    const float bound = (float)L * v;
    int e = 0;
    if (bound > 0.f && __builtin_isfinite(bound)) (void)__builtin_frexpf(bound, &e);
    int sh = 61 - e;
    s_sh = sh < -120 ? -120 : (sh > 120 ? 120 : sh);
  }
  __syncthreads();
  const int sh = FIXED ? s_sh : 0;

  // pass 2: p_t = exp(z_t - max), the sums, and the scatter of p_t cV onto the value atoms
  float m[SM_GMAX], sum[SM_GMAX];
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) {
    m[g] = s_m[g];
    sum[g] = 0.f;
  }
  for (int t = tid; t < L; t += SM_THREADS) {
    const size_t o = cbase + (size_t)t * s;
    float z[SM_GMAX];
    logits(k_idx + o, k_coef + o, s, N, gn, qs, z);
    float p[SM_GMAX];
#pragma unroll
    for (int g = 0; g < SM_GMAX; ++g) {
      p[g] = g < gn ? __expf(z[g] * scale - m[g]) : 0.f;
      sum[g] += p[g];
    }
    for (int k0 = 0; k0 < s; k0 += SM_CH) {
      int vj[SM_CH];
      float vcf[SM_CH];
      load_slots(v_idx + o + k0, v_coef + o + k0, s - k0, (s & 3) == 0, vj, vcf);
#pragma unroll
      for (int k = 0; k < SM_CH; ++k) {
        if (vj[k] >= 0 && vj[k] < N) {
#pragma unroll
          for (int g = 0; g < SM_GMAX; ++g) {
            if (g < gn) {
              if constexpr (FIXED) {
                const long long qv = __double2ll_rn((double)__builtin_ldexpf(p[g] * vcf[k], sh));
                atomicAdd(&wq[g * N + vj[k]], (unsigned long long)qv);
              } else {
                atomicAdd(&wv[g * N + vj[k]], p[g] * vcf[k]);
              }
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) {
    float v = wave_sum(sum[g]);
    if (lane == 0) s_red[wave][g] = v;
  }
  __syncthreads();
  if (tid < SM_GMAX) {
    float v = 0.f;
    for (int w = 0; w < SM_THREADS / 64; ++w) v += s_red[w][tid];
    s_sum[tid] = v;
  }
  __syncthreads();
  // weights / sum over the qd rows (this workgroup owns them); a row without tokens gets 0
  for (int i = tid; i < gn * N; i += SM_THREADS) {
    const float S = s_sum[i / N];
    float wi;
    if constexpr (FIXED) wi = (float)__builtin_ldexp((double)(long long)wq[i], -sh);
    else wi = wv[i];
    rows[i] = S > 0.f ? wi / S : 0.f;
  }
}

// part[range][query][:] = sum_{j in the range} w[query][j] d^V_j.  A workgroup takes
// OUT_QUERIES queries x OUT_ATOMS atoms; 32-atom chunks of w (stored atom-major) and of D_V (as
// fp32) are staged in LDS, and thread (tq, td) accumulates a 4-query x 4-element register tile
// from one 16-byte read of each per atom.
template <int DT, int D>
__global__ __launch_bounds__(256) void attend_out_kernel(const uint8_t *__restrict__ dictV,
                                                         const float *__restrict__ w, int RG,
                                                         int N, float *__restrict__ part_all) {
  constexpr int CK = 32;                  // atoms per staged chunk
  constexpr int QB = OUT_QUERIES;         // 32 queries: 8 thread rows of 4
  constexpr int TD = D / 4;               // thread columns of 4 elements (32 or 16)
  constexpr int TQ = 256 / TD;            // thread rows (8 or 16)
  constexpr int QT = QB / TQ;             // queries per thread (4 or 2)
  __shared__ __attribute__((aligned(16))) float s_w[CK][QB];
  __shared__ __attribute__((aligned(16))) float s_v[CK][D];
  const int tid = threadIdx.x;
  const int tq = tid / TD, td = tid % TD;
  const int q0 = blockIdx.x * QB;
  const int j0 = blockIdx.y * OUT_ATOMS;
  const int j1 = min(N, j0 + OUT_ATOMS);
  float acc[QT][4];
#pragma unroll
  for (int i = 0; i < QT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
  for (int c0 = j0; c0 < j1; c0 += CK) {
    for (int i = tid; i < QB * CK; i += 256) {
      const int qi = i / CK, a = i % CK;
      const int qq = q0 + qi, j = c0 + a;
      s_w[a][qi] = (qq < RG && j < j1) ? w[(size_t)qq * N + j] : 0.f;
    }
    for (int i = tid; i < CK * D; i += 256) {
      const int a = i / D, e = i % D;
      const int j = c0 + a;
      s_v[a][e] = j < j1 ? elem_f<DT>(dictV + (size_t)j * D * Elem<DT>::bytes, e) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int a = 0; a < CK; ++a) {
      float wq[QT];
#pragma unroll
      for (int i = 0; i < QT; ++i) wq[i] = s_w[a][QT * tq + i];
      const float4 dv = *reinterpret_cast<const float4 *>(&s_v[a][4 * td]);
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        acc[i][0] = fmaf(wq[i], dv.x, acc[i][0]);
        acc[i][1] = fmaf(wq[i], dv.y, acc[i][1]);
        acc[i][2] = fmaf(wq[i], dv.z, acc[i][2]);
        acc[i][3] = fmaf(wq[i], dv.w, acc[i][3]);
      }
    }
    __syncthreads();
  }
  float *part = part_all + (size_t)blockIdx.y * RG * D;
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    const int qq = q0 + QT * tq + i;
    if (qq >= RG) continue;
    *reinterpret_cast<float4 *>(&part[(size_t)qq * D + 4 * td]) =
        make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  }
}

// out[i] = sum over the atom ranges of part[range][i]
__global__ __launch_bounds__(256) void attend_reduce_kernel(const float *__restrict__ part,
                                                            int nranges, size_t total,
                                                            float *__restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  float acc = 0.f;
  for (int r = 0; r < nranges; ++r) acc += part[(size_t)r * total + i];
  out[i] = acc;
}

#define FADKV_ATT_INST(DT, D)                                                                  \
  template __global__ void attend_qd_kernel<DT, D>(const uint8_t *, const uint8_t *, int, int, \
                                                   float *);                                  \
  template __global__ void attend_out_kernel<DT, D>(const uint8_t *, const float *, int, int,  \
                                                    float *);
FADKV_ATT_INST(DT_F32, 64)
FADKV_ATT_INST(DT_F32, 128)
FADKV_ATT_INST(DT_F16, 64)
FADKV_ATT_INST(DT_F16, 128)
FADKV_ATT_INST(DT_BF16, 64)
FADKV_ATT_INST(DT_BF16, 128)

hipError_t launch_attend(int dtype, int d, const void *dictK, const void *dictV, int N, int s,
                         const int32_t *k_idx, const float *k_coef, const int32_t *v_idx,
                         const float *v_coef, const int32_t *lens, int R, int T, const void *q,
                         int G, float scale, float *out, float *ws, hipStream_t stream) {
  const int RG = R * G;
  const uint8_t *K = static_cast<const uint8_t *>(dictK);
  const uint8_t *V = static_cast<const uint8_t *>(dictV);
  const uint8_t *Q = static_cast<const uint8_t *>(q);
  dim3 g1((unsigned)((RG + QD_QUERIES - 1) / QD_QUERIES), (unsigned)((N + QD_ATOMS - 1) / QD_ATOMS));
  // queries per softmax workgroup: qd rows and weights of gw queries fit the LDS budget (8-byte
  // fixed-point weights when at least one query fits that way, else fp32 weights)
  const bool fixed = (size_t)N * 12 + 4 <= (size_t)SM_LDS_FIXED;
  int gw = fixed ? (int)((size_t)(SM_LDS_FIXED - 4) / ((size_t)N * 12)) : SM_LDS_FLOATS / (2 * N);
  gw = gw < 1 ? 1 : (gw > SM_GMAX ? SM_GMAX : gw);
  gw = gw > G ? G : gw;
  dim3 g2((unsigned)R, (unsigned)((G + gw - 1) / gw));
  // qd rows (padded to 8 bytes) + weights: <= 156 KB fixed-point / 128 KB fp32
  const size_t lds2 = fixed ? (((size_t)gw * N + 1) & ~(size_t)1) * 4 + (size_t)gw * N * 8
                            : (size_t)gw * N * 8;
  if (lds2 > 65536) {
    const hipError_t e = fixed
        ? hipFuncSetAttribute(reinterpret_cast<const void *>(attend_softmax_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, SM_LDS_FIXED)
        : hipFuncSetAttribute(reinterpret_cast<const void *>(attend_softmax_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(SM_LDS_FLOATS * sizeof(float)));
    if (e != hipSuccess) return e;
  }
  const int nranges = (N + OUT_ATOMS - 1) / OUT_ATOMS;
  dim3 g3((unsigned)((RG + OUT_QUERIES - 1) / OUT_QUERIES), (unsigned)nranges);
  float *part = ws + (size_t)RG * N;          // [nranges][RG][d] partial sums
  const size_t total = (size_t)RG * d;
  dim3 g4((unsigned)((total + 255) / 256));
#define L(DT, D)                                                                                \
  do {                                                                                          \
    hipLaunchKernelGGL((attend_qd_kernel<DT, D>), g1, dim3(256), 0, stream, K, Q, RG, N, ws);    \
    if (fixed)                                                                                  \
      hipLaunchKernelGGL(attend_softmax_kernel<true>, g2, dim3(SM_THREADS), lds2, stream, k_idx, \
                         k_coef, v_idx, v_coef, lens, T, s, N, G, gw, scale, ws);               \
    else                                                                                        \
      hipLaunchKernelGGL(attend_softmax_kernel<false>, g2, dim3(SM_THREADS), lds2, stream, k_idx,\
                         k_coef, v_idx, v_coef, lens, T, s, N, G, gw, scale, ws);               \
    hipLaunchKernelGGL((attend_out_kernel<DT, D>), g3, dim3(256), 0, stream, V, ws, RG, N, part); \
    hipLaunchKernelGGL(attend_reduce_kernel, g4, dim3(256), 0, stream, part, nranges, total, out); \
  } while (0)
  if (dtype == DT_F32) { if (d == 64) L(DT_F32, 64); else L(DT_F32, 128); }
  else if (dtype == DT_F16) { if (d == 64) L(DT_F16, 64); else L(DT_F16, 128); }
  else { if (d == 64) L(DT_BF16, 64); else L(DT_BF16, 128); }
#undef L
  return hipGetLastError();
}

}  // namespace fadkv
