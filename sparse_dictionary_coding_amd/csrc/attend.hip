// Decode attention over sparse-coded keys and values (the consumer of the encoder's codes).
//
// A cached key is k_t = sum_k cK[t][k] d^K_{iK[t][k]}, so <q, k_t> = sum_k cK[t][k] qd[iK[t][k]]
// with qd = D_K q computed once per query, and sum_t p_t v_t = w . D_V with the softmax weights
// scattered onto the value atoms, w[j] = sum_{t,k: iV[t][k] = j} p_t cV[t][k].  Three kernels:
//   attend_qd       qd[query][j] = <q, d^K_j>: v_mfma_f32_16x16x32 (16x16x4 for fp32), 64 queries
//                   x 512 atoms per workgroup; also clears out[]
//   attend_softmax  one workgroup per (row, query group): qd rows in LDS, a max pass and an
//                   exp/sum/scatter pass over the row's tokens (s LDS gathers per token and
//                   query, fp32 LDS atomics onto w), then w / sum written over qd
//   attend_out      out[query] += w[query][j0:j1] . D_V[j0:j1] for 16 queries x 256 atoms per
//                   workgroup (fp32, global atomics across atom ranges)
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
constexpr int QD_ATOMS = 512;      // 32 tiles of 16 atoms, eight per wave
constexpr int SM_THREADS = 256;
constexpr int SM_GMAX = 8;         // queries per softmax workgroup
constexpr int SM_LDS_FLOATS = 32768;   // qd rows + weights: 128 KB
constexpr int OUT_QUERIES = 16;
constexpr int OUT_ATOMS = 256;

}  // namespace

// qd[query][j] = <q[query], d^K_j>; block b of the workgroup's 64 queries is the B operand
// (column = query), each 16-atom tile the A operand (row = atom); lane l holds chunk
// 4 i + l / 16 of row l % 16 on both sides, so the product sums over all of d.
template <int DT, int D>
__global__ __launch_bounds__(256) void attend_qd_kernel(const uint8_t *__restrict__ dictK,
                                                        const uint8_t *__restrict__ Q, int RG,
                                                        int N, float *__restrict__ qd,
                                                        float *__restrict__ out) {
  using G = AGeo<DT, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q0 = blockIdx.x * QD_QUERIES;
  const int r16 = lane & 15, g4 = lane >> 4;
  if (blockIdx.y == 0) {   // out is accumulated by attend_out
    for (int i = threadIdx.x; i < QD_QUERIES * D; i += blockDim.x) {
      const int qq = q0 + i / D;
      if (qq < RG) out[(size_t)qq * D + i % D] = 0.f;
    }
  }
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
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = t * 16 + 4 * g4 + e;
        if (j < N) qd[(size_t)qq * N + j] = acc[k][e];
      }
    }
  }
}

// One workgroup per (row, group of up to SM_GMAX queries).
__global__ __launch_bounds__(SM_THREADS) void attend_softmax_kernel(
    const int32_t *__restrict__ k_idx, const float *__restrict__ k_coef,
    const int32_t *__restrict__ v_idx, const float *__restrict__ v_coef,
    const int32_t *__restrict__ lens, int T, int s, int N, int G, int gw, float scale,
    float *__restrict__ ws) {
  extern __shared__ float s_lds[];
  __shared__ float s_red[SM_THREADS / 64][SM_GMAX];
  __shared__ float s_m[SM_GMAX], s_sum[SM_GMAX];
  const int r = blockIdx.x;
  const int g0 = blockIdx.y * gw;
  const int gn = min(gw, G - g0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int L = lens[r];
  L = L < 0 ? 0 : (L > T ? T : L);
  float *qs = s_lds;                 // [gn][N] qd rows
  float *wv = s_lds + (size_t)gw * N;   // [gn][N] value-atom weights
  float *rows = ws + ((size_t)r * G + g0) * N;
  for (int i = tid; i < gn * N; i += SM_THREADS) {
    qs[i] = rows[i];
    wv[i] = 0.f;
  }
  __syncthreads();
  const size_t cbase = (size_t)r * T * s;

  // pass 1: the largest logit of every query
  float mx[SM_GMAX];
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) mx[g] = -__builtin_inff();
  for (int t = tid; t < L; t += SM_THREADS) {
    float z[SM_GMAX];
#pragma unroll
    for (int g = 0; g < SM_GMAX; ++g) z[g] = 0.f;
    for (int k = 0; k < s; ++k) {
      const int j = k_idx[cbase + (size_t)t * s + k];
      if (j < 0 || j >= N) continue;
      const float c = k_coef[cbase + (size_t)t * s + k];
#pragma unroll
      for (int g = 0; g < SM_GMAX; ++g)
        if (g < gn) z[g] = fmaf(c, qs[g * N + j], z[g]);
    }
#pragma unroll
    for (int g = 0; g < SM_GMAX; ++g) mx[g] = fmaxf(mx[g], z[g] * scale);
  }
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) {
    float v = mx[g];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0) s_red[wave][g] = v;
  }
  __syncthreads();
  if (tid < SM_GMAX) {
    float v = s_red[0][tid];
    for (int w = 1; w < SM_THREADS / 64; ++w) v = fmaxf(v, s_red[w][tid]);
    s_m[tid] = v;
  }
  __syncthreads();

  // pass 2: p_t = exp(z_t - max), the sums, and the scatter of p_t cV onto the value atoms
  float m[SM_GMAX], sum[SM_GMAX];
#pragma unroll
  for (int g = 0; g < SM_GMAX; ++g) {
    m[g] = s_m[g];
    sum[g] = 0.f;
  }
  for (int t = tid; t < L; t += SM_THREADS) {
    float z[SM_GMAX];
#pragma unroll
    for (int g = 0; g < SM_GMAX; ++g) z[g] = 0.f;
    for (int k = 0; k < s; ++k) {
      const int j = k_idx[cbase + (size_t)t * s + k];
      if (j < 0 || j >= N) continue;
      const float c = k_coef[cbase + (size_t)t * s + k];
#pragma unroll
      for (int g = 0; g < SM_GMAX; ++g)
        if (g < gn) z[g] = fmaf(c, qs[g * N + j], z[g]);
    }
    float p[SM_GMAX];
#pragma unroll
    for (int g = 0; g < SM_GMAX; ++g) {
      p[g] = g < gn ? __expf(z[g] * scale - m[g]) : 0.f;
      sum[g] += p[g];
    }
    for (int k = 0; k < s; ++k) {
      const int j = v_idx[cbase + (size_t)t * s + k];
      if (j < 0 || j >= N) continue;
      const float c = v_coef[cbase + (size_t)t * s + k];
#pragma unroll
      for (int g = 0; g < SM_GMAX; ++g)
        if (g < gn) atomicAdd(&wv[g * N + j], p[g] * c);
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
    rows[i] = S > 0.f ? wv[i] / S : 0.f;
  }
}

// out[query][:] += sum_{j in this workgroup's atom range} w[query][j] d^V_j: thread (query
// qi = tid / 16, part dp = tid % 16) owns D / 16 consecutive output elements.
template <int DT, int D>
__global__ __launch_bounds__(256) void attend_out_kernel(const uint8_t *__restrict__ dictV,
                                                         const float *__restrict__ w, int RG,
                                                         int N, float *__restrict__ out) {
  constexpr int DP = D / 16;
  constexpr int ROWB = D * Elem<DT>::bytes;
  const int qq = blockIdx.x * OUT_QUERIES + threadIdx.x / 16;
  const int dp = threadIdx.x % 16;
  if (qq >= RG) return;
  const int j0 = blockIdx.y * OUT_ATOMS;
  const int j1 = min(N, j0 + OUT_ATOMS);
  float acc[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) acc[i] = 0.f;
  const float *wrow = w + (size_t)qq * N;
  for (int j = j0; j < j1; ++j) {
    const float wj = wrow[j];
    const uint8_t *src = dictV + (size_t)j * ROWB + dp * DP * Elem<DT>::bytes;
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] = fmaf(wj, elem_f<DT>(src, i), acc[i]);
  }
#pragma unroll
  for (int i = 0; i < DP; ++i) atomicAdd(&out[(size_t)qq * D + dp * DP + i], acc[i]);
}

#define FADKV_ATT_INST(DT, D)                                                                  \
  template __global__ void attend_qd_kernel<DT, D>(const uint8_t *, const uint8_t *, int, int, \
                                                   float *, float *);                         \
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
  // queries per softmax workgroup: qd rows and weights of gw queries fit the LDS budget
  int gw = SM_LDS_FLOATS / (2 * N);
  gw = gw < 1 ? 1 : (gw > SM_GMAX ? SM_GMAX : gw);
  gw = gw > G ? G : gw;
  dim3 g2((unsigned)R, (unsigned)((G + gw - 1) / gw));
  const size_t lds2 = (size_t)2 * gw * N * sizeof(float);   // <= 128 KB for N <= 16384
  if (lds2 > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(attend_softmax_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(SM_LDS_FLOATS * sizeof(float)));
    if (e != hipSuccess) return e;
  }
  dim3 g3((unsigned)((RG + OUT_QUERIES - 1) / OUT_QUERIES), (unsigned)((N + OUT_ATOMS - 1) / OUT_ATOMS));
#define L(DT, D)                                                                                \
  do {                                                                                          \
    hipLaunchKernelGGL((attend_qd_kernel<DT, D>), g1, dim3(256), 0, stream, K, Q, RG, N, ws, out); \
    hipLaunchKernelGGL(attend_softmax_kernel, g2, dim3(SM_THREADS), lds2, stream, k_idx, k_coef, \
                       v_idx, v_coef, lens, T, s, N, G, gw, scale, ws);                         \
    hipLaunchKernelGGL((attend_out_kernel<DT, D>), g3, dim3(256), 0, stream, V, ws, RG, N, out); \
  } while (0)
  if (dtype == DT_F32) { if (d == 64) L(DT_F32, 64); else L(DT_F32, 128); }
  else if (dtype == DT_F16) { if (d == 64) L(DT_F16, 64); else L(DT_F16, 128); }
  else { if (d == 64) L(DT_BF16, 64); else L(DT_BF16, 128); }
#undef L
  return hipGetLastError();
}

}  // namespace fadkv
