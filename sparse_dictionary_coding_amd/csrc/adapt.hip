// Fixed-size dictionary adaptation (FAD-KV Figure 2), its append-only contrast (abstract,
// Fig. 3a: new atoms go to the next free slots and the dictionary grows) and reconstruction.
//
// Commit of one step, per dictionary, after every vector was encoded against the dictionary as
// it stood at step start:
//   mark    (one thread per row)  : usage[j] += 1 for atoms of non-triggering codes (integer
//                                   atomics: the result does not depend on their order) and
//                                   mark every atom selected by any code of the step;
//   select  (one block per dict)  : rank the triggering rows in row order; list the inactive
//                                   atoms (usage < tau_c, unmarked) in (usage, index) order,
//                                   one usage level at a time, until there is one per trigger;
//   apply   (one wave per row)    : trigger k takes candidate k: the atom becomes x/||x||
//                                   (fp64, rounded to the storage dtype), usage = 1, and the
//                                   row is re-coded onto it with the one-atom ridge coefficient;
//                                   triggers past the list keep their code and commit its usage.
// No step depends on thread scheduling, so the outcome is deterministic.
#include "common.h"
#include "kernels.h"

namespace fadkv {

__global__ void adapt_clear_kernel(uint32_t *__restrict__ words, size_t count) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x)
    words[i] = 0u;
}

__global__ __launch_bounds__(256) void adapt_mark_kernel(const int32_t *__restrict__ idx,
                                                         const uint8_t *__restrict__ flags,
                                                         uint32_t *__restrict__ usage,
                                                         uint8_t *__restrict__ touched,
                                                         int touched_stride, int N, int M, int s,
                                                         size_t G, size_t base) {
  const size_t gv = base + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gv >= G) return;
  const int dict = (int)(gv / (size_t)M);
  const uint8_t fl = flags[gv];
  if (fl & FLAG_NONFINITE) return;
  const bool commit = !(fl & FLAG_TRIGGER);
  for (int k = 0; k < s; ++k) {
    const int j = idx[gv * s + k];
    if (j < 0 || j >= N) continue;
    touched[(size_t)dict * touched_stride + j] = 1;
    if (commit) atomicAdd(&usage[(size_t)dict * N + j], 1u);
  }
}

// The same marks and usage commits for large steps, privatised per workgroup: workgroup b takes
// rows [m0, m1) of dictionary b / chunks, counts its committed slots per atom and its touched
// atoms in LDS (one thread per code slot), then adds every nonzero count to the global
// counter with one atomic.  Integer sums commute, so the counters equal the per-slot
// kernel's.  LDS: N words of counts and N bytes of marks.
constexpr int MARK_THREADS = 256;
constexpr int kMarkLdsMaxN = 12288;   // 48 KB of counts + 12 KB of marks
__global__ __launch_bounds__(MARK_THREADS) void adapt_mark_lds_kernel(
    const int32_t *__restrict__ idx, const uint8_t *__restrict__ flags,
    uint32_t *__restrict__ usage, uint8_t *__restrict__ touched, int touched_stride, int N, int M,
    int s, int chunks) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s_cnt[];
  uint8_t *s_tch = reinterpret_cast<uint8_t *>(s_cnt + N);
  const int dict = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int per = (M + chunks - 1) / chunks;
  const int m0 = c * per, m1 = min(M, m0 + per);
  const int words = N + (N + 3) / 4;
  for (int i = threadIdx.x; i < words; i += MARK_THREADS) s_cnt[i] = 0u;
  __syncthreads();
  const size_t row0 = (size_t)dict * M;
  const long e1 = (long)m1 * s;
  for (long e = (long)m0 * s + threadIdx.x; e < e1; e += MARK_THREADS) {
    const int m = (int)(e / s);
    const uint8_t fl = flags[row0 + m];
    if (fl & FLAG_NONFINITE) continue;
    const int j = idx[row0 * s + e];
    if (j < 0 || j >= N) continue;
    s_tch[j] = 1;
    if (!(fl & FLAG_TRIGGER)) atomicAdd(&s_cnt[j], 1u);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < N; j += MARK_THREADS) {
    const uint32_t v = s_cnt[j];
    if (v) atomicAdd(&usage[(size_t)dict * N + j], v);
    if (s_tch[j]) touched[(size_t)dict * touched_stride + j] = 1;
  }
}

namespace {
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

// exclusive prefix count of `pred` over the block in thread order; returns the total
__device__ __forceinline__ int block_prefix(bool pred, int *s_w, int &prefix) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long mask = __ballot(pred);
  const int below = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) s_w[wave] = __popcll(mask);
  __syncthreads();
  int before = 0, total = 0;
  for (int q = 0; q < SEL_WAVES; ++q) {
    const int c = s_w[q];
    before += q < wave ? c : 0;
    total += c;
  }
  __syncthreads();
  prefix = before + below;
  return total;
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t *s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t w = __shfl_xor(v, o, 64);
    v = w < v ? w : v;
  }
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  uint32_t m = s_w[0];
  for (int q = 1; q < SEL_WAVES; ++q) m = s_w[q] < m ? s_w[q] : m;
  __syncthreads();
  return m;
}
}  // namespace

// n_atoms == nullptr: fixed size (inactive atoms are the candidates).  Otherwise append-only
// growth: dictionary `dict` uses slots [0, n_atoms[dict]) of its capacity N, the candidates are
// the next free slots in order, and n_atoms[dict] grows by the number handed out.
__global__ __launch_bounds__(SEL_THREADS) void adapt_select_kernel(
    const uint32_t *__restrict__ usage, const uint8_t *__restrict__ touched, int touched_stride,
    const uint8_t *__restrict__ flags, int N, int M, uint32_t tau_c, int32_t *__restrict__ rank,
    int32_t *__restrict__ cand, int32_t *__restrict__ ccount, int32_t *__restrict__ n_atoms) {
  __shared__ int s_w[SEL_WAVES];
  __shared__ uint32_t s_u[SEL_WAVES];
  const int dict = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row0 = (size_t)dict * M;

  int T = 0;
  for (int m0 = 0; m0 < M; m0 += SEL_THREADS) {
    const int m = m0 + tid;
    const bool t = m < M && (flags[row0 + m] & FLAG_TRIGGER);
    int prefix;
    const int total = block_prefix(t, s_w, prefix);
    if (m < M) rank[row0 + m] = t ? T + prefix : -1;
    T += total;
  }

  if (n_atoms) {
    int n0 = n_atoms[dict];
    n0 = n0 < 0 ? 0 : (n0 > N ? N : n0);
    const int take = T < N - n0 ? T : N - n0;
    for (int k = tid; k < take; k += SEL_THREADS) cand[row0 + k] = n0 + k;
    __syncthreads();   // every thread has read n_atoms[dict]
    if (tid == 0) {
      ccount[dict] = take;
      n_atoms[dict] = n0 + take;
    }
    return;
  }

  const uint32_t *u = usage + (size_t)dict * N;
  const uint8_t *tch = touched + (size_t)dict * touched_stride;
  int count = 0;
  unsigned long long floor_u = 0;   // usage levels below this are exhausted
  while (count < T && floor_u < tau_c) {
    uint32_t mine = 0xffffffffu;
    for (int j = tid; j < N; j += SEL_THREADS) {
      const uint32_t uj = u[j];
      if (uj < tau_c && uj >= floor_u && !tch[j]) mine = uj < mine ? uj : mine;
    }
    const uint32_t level = block_min_u32(mine, s_u);
    if (level == 0xffffffffu) break;
    for (int j0 = 0; j0 < N && count < T; j0 += SEL_THREADS) {
      const int j = j0 + tid;
      const bool c = j < N && u[j] == level && !tch[j];
      int prefix;
      const int total = block_prefix(c, s_w, prefix);
      if (c && count + prefix < T) cand[row0 + count + prefix] = j;
      count += total;
    }
    floor_u = (unsigned long long)level + 1ull;
  }
  if (tid == 0) ccount[dict] = count < T ? count : T;
}

// The replacement of one triggering row by one wave: the atom row becomes x/||x|| (fp64,
// rounded to the storage dtype) and the row's code the single new atom with the one-atom ridge
// coefficient c = <a, x> / ((1 + ridge_rel) <a, a> + ridge_abs); e = ||x - c a|| / ||x||.
template <int DT, int D>
__device__ __forceinline__ void recode_onto_new_atom(uint8_t *__restrict__ arow,
                                                     const uint8_t *__restrict__ xr,
                                                     float ridge_abs, float ridge_rel, int lane,
                                                     float &c_out, float &e_out) {
  constexpr int PER = D / 64;   // elements per lane
  double x[PER];
  double ss = 0.0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    x[p] = (double)elem_f<DT>(xr, lane + 64 * p);
    ss += x[p] * x[p];
  }
  const double nrm = __builtin_sqrt(wave_sum_d(ss));
  double a[PER];
  double g = 0.0, ax = 0.0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int i = lane + 64 * p;
    const uint32_t bits = double_to_storage_bits<DT>(x[p] / nrm);
    if constexpr (DT == DT_F32) {
      reinterpret_cast<uint32_t *>(arow)[i] = bits;
      a[p] = (double)__uint_as_float(bits);
    } else {
      reinterpret_cast<uint16_t *>(arow)[i] = (uint16_t)bits;
      a[p] = (double)(DT == DT_F16 ? f16_bits_to_float(bits) : bf16_bits_to_float(bits));
    }
    g += a[p] * a[p];
    ax += a[p] * x[p];
  }
  g = wave_sum_d(g);
  ax = wave_sum_d(ax);
  const double c = ax / ((1.0 + (double)ridge_rel) * g + (double)ridge_abs);
  double rr = 0.0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const double d = x[p] - c * a[p];
    rr += d * d;
  }
  rr = wave_sum_d(rr);
  c_out = (float)c;
  e_out = (float)(__builtin_sqrt(rr) / nrm);
}

template <int DT, int D>
__global__ __launch_bounds__(256) void adapt_apply_kernel(
    uint8_t *__restrict__ atoms, uint32_t *__restrict__ usage, const uint8_t *__restrict__ X, int N,
    int M, int s, float ridge_abs, float ridge_rel, const int32_t *__restrict__ rank,
    const int32_t *__restrict__ cand, const int32_t *__restrict__ ccount, int32_t *__restrict__ idx,
    float *__restrict__ coef, float *__restrict__ relerr, uint8_t *__restrict__ flags,
    int32_t *__restrict__ replaced, size_t G, size_t base) {
  constexpr int ROWB = D * Elem<DT>::bytes;
  const int lane = threadIdx.x & 63;
  const size_t gv = base + (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gv >= G) return;
  const int dict = (int)(gv / (size_t)M);
  const int r = rank[gv];
  if (r < 0) {
    if (lane == 0) replaced[gv] = -1;
    return;
  }
  if (r < ccount[dict]) {
    const int j = cand[(size_t)dict * M + r];
    float c, e;
    recode_onto_new_atom<DT, D>(atoms + ((size_t)dict * N + j) * ROWB, X + gv * ROWB, ridge_abs,
                                ridge_rel, lane, c, e);
    if (lane < s) {
      idx[gv * s + lane] = lane == 0 ? j : -1;
      coef[gv * s + lane] = lane == 0 ? c : 0.f;
    }
    if (lane == 0) {
      usage[(size_t)dict * N + j] = 1u;
      relerr[gv] = e;
      flags[gv] = flags[gv] | FLAG_REPLACED;
      replaced[gv] = j;
    }
  } else {
    if (lane < s) {
      const int jj = idx[gv * s + lane];
      if (jj >= 0 && jj < N) atomicAdd(&usage[(size_t)dict * N + jj], 1u);
    }
    if (lane == 0) {
      flags[gv] = flags[gv] | FLAG_EXHAUSTED;
      replaced[gv] = -1;
    }
  }
}


// The whole commit of one dictionary in one workgroup, for steps of at most FUSED_MAXM rows
// and dictionaries of at most FUSED_MAXN atoms (decode steps): the dictionary's usage counters
// and touched marks live in LDS, and mark, rank, candidate listing and apply run as phases of
// one kernel with the same rules (and results) as the separate kernels above.
constexpr int FUSED_MAXN = 16384;
constexpr int FUSED_MAXM = 4096;

template <int DT, int D>
__global__ __launch_bounds__(SEL_THREADS) void adapt_fused_kernel(
    uint8_t *__restrict__ atoms, uint32_t *__restrict__ usage, const uint8_t *__restrict__ X,
    int N, int M, int s, float ridge_abs, float ridge_rel, uint32_t tau_c,
    int32_t *__restrict__ idx, float *__restrict__ coef, float *__restrict__ relerr,
    uint8_t *__restrict__ flags, int32_t *__restrict__ replaced, int32_t *__restrict__ n_atoms) {
  constexpr int ROWB = D * Elem<DT>::bytes;
  __shared__ uint32_t s_u[FUSED_MAXN];
  __shared__ uint8_t s_t[FUSED_MAXN];
  __shared__ int s_trig[FUSED_MAXM];
  __shared__ int s_cand[FUSED_MAXM];
  __shared__ int s_w[SEL_WAVES];
  __shared__ uint32_t s_m[SEL_WAVES];
  const int dict = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row0 = (size_t)dict * M;
  uint32_t *ug = usage + (size_t)dict * N;

  for (int j = tid; j < N; j += SEL_THREADS) {
    s_u[j] = ug[j];
    s_t[j] = 0;
  }
  __syncthreads();
  // mark: every atom of every code is touched; non-triggering codes commit their usage
  for (int e = tid; e < M * s; e += SEL_THREADS) {
    const int m = e / s;
    const uint8_t fl = flags[row0 + m];
    if (fl & FLAG_NONFINITE) continue;
    const int j = idx[row0 * s + e];
    if (j < 0 || j >= N) continue;
    s_t[j] = 1;
    if (!(fl & FLAG_TRIGGER)) atomicAdd(&s_u[j], 1u);
  }
  // triggering rows in row order
  int T = 0;
  for (int m0 = 0; m0 < M; m0 += SEL_THREADS) {
    const int m = m0 + tid;
    const bool t = m < M && (flags[row0 + m] & FLAG_TRIGGER);
    int prefix;
    const int total = block_prefix(t, s_w, prefix);   // its barrier also closes the mark phase
    if (t) s_trig[T + prefix] = m;
    T += total;
  }
  // candidates: the next free slots (append-only growth) or the inactive atoms in (usage, index)
  // order, one usage level at a time
  int count = 0;
  if (n_atoms) {
    int n0 = n_atoms[dict];
    n0 = n0 < 0 ? 0 : (n0 > N ? N : n0);
    count = T < N - n0 ? T : N - n0;
    for (int k = tid; k < count; k += SEL_THREADS) s_cand[k] = n0 + k;
    __syncthreads();   // every thread has read n_atoms[dict]
    if (tid == 0) n_atoms[dict] = n0 + count;
  } else {
    unsigned long long floor_u = 0;
    while (count < T && floor_u < tau_c) {
      uint32_t mine = 0xffffffffu;
      for (int j = tid; j < N; j += SEL_THREADS) {
        const uint32_t uj = s_u[j];
        if (uj < tau_c && uj >= floor_u && !s_t[j]) mine = uj < mine ? uj : mine;
      }
      const uint32_t level = block_min_u32(mine, s_m);
      if (level == 0xffffffffu) break;
      for (int j0 = 0; j0 < N && count < T; j0 += SEL_THREADS) {
        const int j = j0 + tid;
        const bool c = j < N && s_u[j] == level && !s_t[j];
        int prefix;
        const int total = block_prefix(c, s_w, prefix);
        if (c && count + prefix < T) s_cand[count + prefix] = j;
        count += total;
      }
      floor_u = (unsigned long long)level + 1ull;
    }
    count = count < T ? count : T;
  }
  __syncthreads();
  for (int m = tid; m < M; m += SEL_THREADS)
    if (!(flags[row0 + m] & FLAG_TRIGGER)) replaced[row0 + m] = -1;
  // apply: one wave per triggering row
  for (int k = wave; k < T; k += SEL_WAVES) {
    const size_t gv = row0 + s_trig[k];
    if (k < count) {
      const int j = s_cand[k];
      float c, e;
      recode_onto_new_atom<DT, D>(atoms + ((size_t)dict * N + j) * ROWB, X + gv * ROWB,
                                  ridge_abs, ridge_rel, lane, c, e);
      if (lane < s) {
        idx[gv * s + lane] = lane == 0 ? j : -1;
        coef[gv * s + lane] = lane == 0 ? c : 0.f;
      }
      if (lane == 0) {
        s_u[j] = 1u;
        relerr[gv] = e;
        flags[gv] = flags[gv] | FLAG_REPLACED;
        replaced[gv] = j;
      }
    } else {
      if (lane < s) {
        const int jj = idx[gv * s + lane];
        if (jj >= 0 && jj < N) atomicAdd(&s_u[jj], 1u);
      }
      if (lane == 0) {
        flags[gv] = flags[gv] | FLAG_EXHAUSTED;
        replaced[gv] = -1;
      }
    }
  }
  __syncthreads();
  for (int j = tid; j < N; j += SEL_THREADS) ug[j] = s_u[j];
}

template <int DT, int D, int ODT>
__global__ __launch_bounds__(256) void reconstruct_kernel(const uint8_t *__restrict__ atoms,
                                                          const int32_t *__restrict__ idx,
                                                          const float *__restrict__ coef, int N,
                                                          int M, int s, uint8_t *__restrict__ out,
                                                          size_t G, size_t base) {
  constexpr int ROWB = D * Elem<DT>::bytes;
  const size_t e = base + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t gv = e / D;
  const int i = (int)(e % D);
  if (gv >= G) return;
  const int dict = (int)(gv / (size_t)M);
  float acc = 0.f;
  for (int k = 0; k < s; ++k) {
    const int j = idx[gv * s + k];
    if (j < 0 || j >= N) continue;
    acc = fmaf(coef[gv * s + k], elem_f<DT>(atoms + ((size_t)dict * N + j) * ROWB, i), acc);
  }
  if constexpr (ODT == DT_F32) reinterpret_cast<float *>(out)[e] = acc;
  else if constexpr (ODT == DT_F16) reinterpret_cast<uint16_t *>(out)[e] = (uint16_t)float_to_f16_bits(acc);
  else reinterpret_cast<uint16_t *>(out)[e] = (uint16_t)float_to_bf16_bits(acc);
}

hipError_t launch_adapt(int dtype, int d, void *atoms, uint32_t *usage, const void *X, int num_dicts,
                        int N, int M, int s, float ridge_abs, float ridge_rel, uint32_t tau_c,
                        int32_t *idx, float *coef, float *relerr, uint8_t *flags,
                        int32_t *replaced, uint8_t *touched, int touched_stride, int32_t *rank,
                        int32_t *cand, int32_t *ccount, int32_t *n_atoms, hipStream_t stream) {
  const size_t G = (size_t)num_dicts * M;
  uint8_t *A = static_cast<uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
  if (M <= FUSED_MAXM && N <= FUSED_MAXN) {
#define LF(DT, D)                                                                                  \
  hipLaunchKernelGGL((adapt_fused_kernel<DT, D>), dim3(num_dicts), dim3(SEL_THREADS), 0, stream, A, \
                     usage, Xb, N, M, s, ridge_abs, ridge_rel, tau_c, idx, coef, relerr, flags,   \
                     replaced, n_atoms)
    if (dtype == DT_F32) { if (d == 64) LF(DT_F32, 64); else LF(DT_F32, 128); }
    else if (dtype == DT_F16) { if (d == 64) LF(DT_F16, 64); else LF(DT_F16, 128); }
    else { if (d == 64) LF(DT_BF16, 64); else LF(DT_BF16, 128); }
#undef LF
    return hipGetLastError();
  }
  const size_t words = (size_t)num_dicts * touched_stride / 4;
  hipLaunchKernelGGL(adapt_clear_kernel, dim3((unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096)),
                     dim3(256), 0, stream, reinterpret_cast<uint32_t *>(touched), words);
  if (N <= kMarkLdsMaxN) {
    // about 512 workgroups over the step, at least 1024 rows each
    int chunks = (512 + num_dicts - 1) / num_dicts;
    const int by_rows = (M + 1023) / 1024;
    chunks = chunks < by_rows ? chunks : by_rows;
    chunks = chunks < 1 ? 1 : chunks;
    const size_t lds = ((size_t)N + (N + 3) / 4) * sizeof(uint32_t);
    hipLaunchKernelGGL(adapt_mark_lds_kernel, dim3((unsigned)(num_dicts * chunks)),
                       dim3(MARK_THREADS), lds, stream, idx, flags, usage, touched, touched_stride,
                       N, M, s, chunks);
  } else {
    const size_t blocks = (G + 255) / 256;
    for (size_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
      const size_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
      hipLaunchKernelGGL(adapt_mark_kernel, dim3((unsigned)nb), dim3(256), 0, stream, idx, flags,
                         usage, touched, touched_stride, N, M, s, G, b0 * 256);
    }
  }
  hipLaunchKernelGGL(adapt_select_kernel, dim3(num_dicts), dim3(SEL_THREADS), 0, stream, usage,
                     touched, touched_stride, flags, N, M, tau_c, rank, cand, ccount, n_atoms);
  const size_t blocks = (G + 3) / 4;
  for (size_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
    const dim3 grid((unsigned)nb), block(256);
#define L(DT, D)                                                                                   \
  hipLaunchKernelGGL((adapt_apply_kernel<DT, D>), grid, block, 0, stream, A, usage, Xb, N, M, s,  \
                     ridge_abs, ridge_rel, rank, cand, ccount, idx, coef, relerr, flags, replaced, G, \
                     b0 * 4)
    if (dtype == DT_F32) { if (d == 64) L(DT_F32, 64); else L(DT_F32, 128); }
    else if (dtype == DT_F16) { if (d == 64) L(DT_F16, 64); else L(DT_F16, 128); }
    else { if (d == 64) L(DT_BF16, 64); else L(DT_BF16, 128); }
#undef L
  }
  return hipGetLastError();
}

hipError_t launch_reconstruct(int dtype, int d, const void *atoms, const int32_t *idx,
                              const float *coef, int num_dicts, int N, int M, int s, void *out,
                              int out_dtype, hipStream_t stream) {
  const size_t G = (size_t)num_dicts * M;
  const size_t E = G * d;
  const size_t blocks = (E + 255) / 256;
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  uint8_t *O = static_cast<uint8_t *>(out);
  for (size_t b0 = 0; b0 < blocks; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = blocks - b0 < kMaxBlocksPerLaunch ? blocks - b0 : kMaxBlocksPerLaunch;
    const dim3 grid((unsigned)nb), block(256);
#define L(DT, D, ODT) \
  hipLaunchKernelGGL((reconstruct_kernel<DT, D, ODT>), grid, block, 0, stream, A, idx, coef, N, M, s, O, G, b0 * 256)
#define LO(DT, D) do { if (out_dtype == DT_F32) L(DT, D, DT_F32); else if (out_dtype == DT_F16) L(DT, D, DT_F16); else L(DT, D, DT_BF16); } while (0)
#define LD(DT) do { if (d == 64) LO(DT, 64); else LO(DT, 128); } while (0)
    if (dtype == DT_F32) LD(DT_F32);
    else if (dtype == DT_F16) LD(DT_F16);
    else LD(DT_BF16);
#undef LD
#undef LO
#undef L
  }
  return hipGetLastError();
}

}  // namespace fadkv
