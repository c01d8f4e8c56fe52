// Screening scores and exact Top-n candidate pool (FAD-KV abstract and Figure 1: one pass of
// dictionary correlations, then a one-shot Top-n pool by |score|, ties to the lowest index).
//
// One workgroup = 8 waves = one dictionary x 32 vectors.  The 32 vectors are the B operand of
// v_mfma_f32_32x32x{16,2}: they stay in registers for the whole dictionary sweep.  Each wave
// streams its own 32-atom tiles (A operand) from global memory/L2, loading the next tile's
// fragment while the current one is scored; a tile's 32x32 fp32 scores land in 16 accumulators
// per lane, all belonging to the lane's vector (column lane % 32), so every score is handled by
// the lane that owns its vector.  Workgroups are numbered so that all workgroups of one
// dictionary land on the same XCD (dispatch is round-robin over the 8 XCDs).
//
// Selection is an exact radix select on the 47-bit key K = (bits(|score|) << 16) |
// (0xFFFF - atom): larger K = larger |score|, then lower index, and every K is unique.
//   sweep 1: histogram of |score| in 512 bins of 1/32 octave below ~1.5 ||x|| (two 16-bit
//            counters per LDS word); the bin holding the n-th largest key is the boundary;
//   sweep 2: keys above the boundary bin go straight to the pool, keys inside it go to an LDS
//            buffer of CAP entries from which the `need` largest keys are taken.
// A vector whose boundary bin holds more than CAP keys is refined by further sweeps that
// histogram its key range uniformly (256 bins each) until the boundary bin fits.  Every sweep
// recomputes the scores with the MFMA (bit-identical), so scores never leave the chip.
#include "common.h"
#include "kernels.h"

namespace fadkv {

namespace {

constexpr int VT = 32;          // vectors per workgroup (one MFMA column block)
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int BINS0 = 512;      // first-level bins (1/32 octave), two per 32-bit word
constexpr int HW = BINS0 / 2 + 1;   // words per vector histogram row, padded against conflicts
constexpr int RBINS = 256;      // refinement bins (one 32-bit counter per word)
constexpr int CAP = 128;        // boundary-bin capacity per vector
constexpr int TPV = THREADS / VT;   // threads per vector in the histogram scans (16)
constexpr int SHIFT0 = 18;      // key >> 18 = 8 exponent bits + 5 mantissa bits
constexpr int TOP0 = 492;       // bin holding |score| ~ ||x||; 19 bins (~1.5x) above it

enum { ST_IDLE = 0, ST_HIST0, ST_COLLECT, ST_REFINE, ST_RCOLLECT };
enum { PASS_HIST0 = 0, PASS_COLLECT = 1, PASS_GENERIC = 2 };

typedef unsigned long long u64;

template <int DT, int D> struct Geo {
  static constexpr int ROWB = D * Elem<DT>::bytes;   // bytes per row
  static constexpr int HALFB = ROWB / 2;             // bytes per lane (half a row)
  static constexpr int U4 = HALFB / 16;              // 16-byte chunks per lane fragment
};

// 32x32 tile of scores: A = 32 atoms (row = lane % 32), B = 32 vectors (column = lane % 32).
// Lane half h = lane / 32 supplies elements [h * D/2, (h+1) * D/2) of its row; k-slots are
// consumed in the same order on A and B, so the sum runs over all D elements.
template <int DT, int D>
__device__ __forceinline__ float16_t tile_scores(const uint4 (&a)[Geo<DT, D>::U4],
                                                 const uint4 (&b)[Geo<DT, D>::U4]) {
  float16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int i = 0; i < Geo<DT, D>::U4; ++i) {
    if constexpr (DT == DT_F16) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a[i]),
                                                   __builtin_bit_cast(half8_t, b[i]), acc, 0, 0, 0);
    } else if constexpr (DT == DT_BF16) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[i]),
                                                    __builtin_bit_cast(bf16x8_t, b[i]), acc, 0, 0, 0);
    } else {
      const float *fa = reinterpret_cast<const float *>(&a[i]);
      const float *fb = reinterpret_cast<const float *>(&b[i]);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[c], fb[c], acc, 0, 0, 0);
    }
  }
  return acc;
}

// fragment of row `row` (zeros past N): half h of the row, U4 chunks of 16 bytes
template <int DT, int D>
__device__ __forceinline__ void load_frag(const uint8_t *base, int row, int N, int h,
                                          uint4 (&a)[Geo<DT, D>::U4]) {
  using G = Geo<DT, D>;
  const bool ok = row < N;
  const uint4 *src = reinterpret_cast<const uint4 *>(base + (size_t)(ok ? row : 0) * G::ROWB +
                                                     h * G::HALFB);
#pragma unroll
  for (int i = 0; i < G::U4; ++i) a[i] = ok ? src[i] : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ u64 comp_key(uint32_t key31, int atom) {
  return ((u64)key31 << 16) | (u64)(0xFFFFu - (uint32_t)atom);
}

struct LaneState {          // the state of the lane's vector during one sweep
  bool active;
  int state;
  int base;                 // level-0 bin offset
  uint32_t lo32, hi32;      // boundary bin in 31-bit key space (level 0)
  u64 lo, hi;               // boundary range in composite-key space (refinement)
  int shift;
};

struct Shared {
  uint32_t *hist;
  float *bsig;
  int *bidx;
  int *above;
  int *bcnt;
};

// one sweep over the dictionary; PASS selects what every score of an active lane does
template <int DT, int D, int PASS>
__device__ __forceinline__ void sweep(const uint8_t *dict_atoms, int N, int n, int wave, int col,
                                      int h, const uint4 (&b)[Geo<DT, D>::U4], const LaneState &ls,
                                      const Shared &sh, uint16_t *pidx, float *psig) {
  using G = Geo<DT, D>;
  const int ntiles = (N + 31) / 32;
  uint4 a[G::U4], an[G::U4];
  if (wave < ntiles) load_frag<DT, D>(dict_atoms, wave * 32 + col, N, h, a);
  for (int t = wave; t < ntiles; t += WAVES) {
    const bool more = t + WAVES < ntiles;
    if (more) load_frag<DT, D>(dict_atoms, (t + WAVES) * 32 + col, N, h, an);
    const float16_t acc = tile_scores<DT, D>(a, b);
    if (ls.active) {
      const bool full = t * 32 + 32 <= N;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int atom = t * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (!full && atom >= N) continue;
        const float sc = acc[r];
        const uint32_t key = __float_as_uint(sc) & 0x7fffffffu;
        if constexpr (PASS == PASS_HIST0) {
          int bin = (int)(key >> SHIFT0) - ls.base;
          bin = bin < 0 ? 0 : (bin > BINS0 - 1 ? BINS0 - 1 : bin);
          atomicAdd(&sh.hist[col * HW + (bin >> 1)], 1u << ((bin & 1) << 4));
        } else if constexpr (PASS == PASS_COLLECT) {
          if (key >= ls.hi32) {
            const int pos = atomicAdd(&sh.above[col], 1);
            if (pos < n) {
              pidx[pos] = (uint16_t)atom;
              psig[pos] = sc;
            }
          } else if (key >= ls.lo32) {
            const int pos = atomicAdd(&sh.bcnt[col], 1);
            if (pos < CAP) {
              sh.bsig[col * CAP + pos] = sc;
              sh.bidx[col * CAP + pos] = atom;
            }
          }
        } else {
          const u64 K = comp_key(key, atom);
          if (ls.state == ST_REFINE) {
            if (K >= ls.lo && K < ls.hi)
              atomicAdd(&sh.hist[col * HW + (int)((K - ls.lo) >> ls.shift)], 1u);
          } else if (K >= ls.hi) {
            const int pos = atomicAdd(&sh.above[col], 1);
            if (pos < n) {
              pidx[pos] = (uint16_t)atom;
              psig[pos] = sc;
            }
          } else if (K >= ls.lo) {
            const int pos = atomicAdd(&sh.bcnt[col], 1);
            if (pos < CAP) {
              sh.bsig[col * CAP + pos] = sc;
              sh.bidx[col * CAP + pos] = atom;
            }
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < G::U4; ++i) a[i] = an[i];
    }
  }
}

}  // namespace

template <int DT, int D>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void score_topn_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int num_dicts, int N, int M,
    int n, uint16_t *__restrict__ pool_idx, float *__restrict__ pool_sig,
    uint8_t *__restrict__ vstat) {
  using G = Geo<DT, D>;
  __shared__ uint32_t hist[VT * HW];
  __shared__ float bsig[VT * CAP];
  __shared__ int bidx[VT * CAP];
  __shared__ u64 s_lo[VT], s_hi[VT];
  __shared__ uint32_t s_lo32[VT], s_hi32[VT];
  __shared__ int s_state[VT], s_need[VT], s_base[VT], s_shift[VT], s_above[VT], s_bcnt[VT];
  __shared__ int s_busy;

  // workgroup i runs on XCD i % 8; its r-th workgroup takes dictionary x + 8 * (r / B)
  const int nvb = (M + VT - 1) / VT;
  const int xcd = blockIdx.x % 8, rr = blockIdx.x / 8;
  const int dict = xcd + 8 * (rr / nvb);
  if (dict >= num_dicts) return;
  const int v0 = (rr % nvb) * VT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const uint8_t *dict_atoms = atoms + (size_t)dict * N * G::ROWB;
  const size_t vbase = (size_t)dict * M + v0;
  const Shared sh{hist, bsig, bidx, s_above, s_bcnt};

  if (tid < VT) {
    int state = ST_IDLE;
    if (v0 + tid < M) {
      const uint8_t *xr = X + (vbase + tid) * G::ROWB;
      float ss = 0.f;
      bool fin = true;
      for (int i = 0; i < D; ++i) {
        const float f = elem_f<DT>(xr, i);
        fin = fin && __builtin_isfinite(f);
        ss += f * f;
      }
      const uint8_t st = !fin ? VS_NONFINITE : (ss == 0.f ? VS_ZERO : VS_NORMAL);
      vstat[vbase + tid] = st;
      if (st == VS_NORMAL) {
        state = ST_HIST0;
        s_base[tid] = (int)(__float_as_uint(sqrtf(ss)) >> SHIFT0) - TOP0;
      }
    }
    s_state[tid] = state;
    s_need[tid] = n;
    s_above[tid] = 0;
    s_bcnt[tid] = 0;
  }
  uint4 b[G::U4];
  {
    const bool ok = v0 + col < M;
    const uint4 *src = reinterpret_cast<const uint4 *>(X + (vbase + (ok ? col : 0)) * G::ROWB +
                                                       h * G::HALFB);
#pragma unroll
    for (int i = 0; i < G::U4; ++i) b[i] = ok ? src[i] : make_uint4(0, 0, 0, 0);
  }
  for (int i = tid; i < VT * HW; i += THREADS) hist[i] = 0u;
  __syncthreads();

  uint16_t *pidx = pool_idx + (vbase + col) * (size_t)n;
  float *psig = pool_sig + (vbase + col) * (size_t)n;

  // ---- sweep 1: level-0 histogram -----------------------------------------------------------
  {
    LaneState ls{};
    ls.active = s_state[col] == ST_HIST0;
    ls.base = s_base[col];
    sweep<DT, D, PASS_HIST0>(dict_atoms, N, n, wave, col, h, b, ls, sh, pidx, psig);
  }
  __syncthreads();
  {
    // TPV threads per vector: thread `sub` covers bins [32 sub, 32 sub + 32); a suffix sum
    // of the per-thread counts locates the bin holding the n-th largest key
    const int v = tid / TPV, sub = tid % TPV;
    const bool on = s_state[v] == ST_HIST0;
    uint32_t part = 0;
    if (on) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t w = hist[v * HW + 16 * sub + q];
        part += (w & 0xffffu) + (w >> 16);
      }
    }
    uint32_t suf = part;
#pragma unroll
    for (int o = 1; o < TPV; o <<= 1) {
      const uint32_t other = __shfl_down(suf, o, TPV);
      if (sub + o < TPV) suf += other;
    }
    const uint32_t need = (uint32_t)n;
    if (on && suf - part < need && suf >= need) {
      uint32_t above = suf - part, cnt = 0;
      int bstar = 32 * sub;
      for (int bin = 32 * sub + 31; bin >= 32 * sub; --bin) {
        const uint32_t c = (hist[v * HW + (bin >> 1)] >> ((bin & 1) << 4)) & 0xffffu;
        if (above + c >= need) {
          bstar = bin;
          cnt = c;
          break;
        }
        above += c;
      }
      const long long bs = (long long)s_base[v] + bstar;
      long long lob = bstar == 0 ? 0 : bs << SHIFT0;
      long long hib = bstar == BINS0 - 1 ? (1ll << 31) : (bs + 1) << SHIFT0;
      lob = lob < 0 ? 0 : (lob > (1ll << 31) ? (1ll << 31) : lob);
      hib = hib < 0 ? 0 : (hib > (1ll << 31) ? (1ll << 31) : hib);
      s_need[v] = (int)(need - above);
      s_lo32[v] = (uint32_t)lob;
      s_hi32[v] = (uint32_t)(hib > 0x7fffffffll ? 0xffffffffll : hib);
      s_lo[v] = (u64)lob << 16;
      s_hi[v] = (u64)hib << 16;
      if (cnt <= (uint32_t)CAP) {
        s_state[v] = ST_COLLECT;
      } else {
        const u64 width = ((u64)hib - (u64)lob) << 16;
        const int bl = 64 - __clzll(width - 1);
        s_shift[v] = bl > 8 ? bl - 8 : 0;
        s_state[v] = ST_REFINE;
      }
    }
  }
  __syncthreads();

  // ---- sweep 2: collect for every vector whose boundary bin fits -----------------------------
  {
    LaneState ls{};
    ls.active = s_state[col] == ST_COLLECT;
    ls.lo32 = s_lo32[col];
    ls.hi32 = s_hi32[col];
    sweep<DT, D, PASS_COLLECT>(dict_atoms, N, n, wave, col, h, b, ls, sh, pidx, psig);
  }
  __syncthreads();

  // ---- resolve boundaries; refine the rest (rare) -------------------------------------------
  for (int pass = 0;; ++pass) {
    // vectors that collected this pass: take the `need` largest keys of the boundary bin
    for (int slot = tid; slot < VT * CAP; slot += THREADS) {
      const int v = slot / CAP, e = slot % CAP;
      const int st = s_state[v];
      const int cnt = s_bcnt[v] < CAP ? s_bcnt[v] : CAP;
      if ((st != ST_COLLECT && st != ST_RCOLLECT) || e >= cnt) continue;
      const u64 Ke = comp_key(__float_as_uint(bsig[v * CAP + e]) & 0x7fffffffu, bidx[v * CAP + e]);
      int rank = 0;
      for (int q = 0; q < cnt; ++q) {
        const u64 Kq = comp_key(__float_as_uint(bsig[v * CAP + q]) & 0x7fffffffu, bidx[v * CAP + q]);
        rank += Kq > Ke;
      }
      const int need = s_need[v];
      if (rank < need && need <= n) {
        const size_t row = (vbase + v) * (size_t)n;
        const int pos = n - need + rank;
        pool_idx[row + pos] = (uint16_t)bidx[v * CAP + e];
        pool_sig[row + pos] = bsig[v * CAP + e];
      }
    }
    __syncthreads();
    {
      // refinement finalize: TPV threads per vector over RBINS bins
      const int v = tid / TPV, sub = tid % TPV;
      const int st = s_state[v];
      uint32_t part = 0;
      if (st == ST_REFINE && pass > 0) {
#pragma unroll
        for (int q = 0; q < RBINS / TPV; ++q) part += hist[v * HW + (RBINS / TPV) * sub + q];
      }
      uint32_t suf = part;
#pragma unroll
      for (int o = 1; o < TPV; o <<= 1) {
        const uint32_t other = __shfl_down(suf, o, TPV);
        if (sub + o < TPV) suf += other;
      }
      if (sub == 0 && (st == ST_COLLECT || st == ST_RCOLLECT)) s_state[v] = ST_IDLE;
      const uint32_t need = (uint32_t)s_need[v];
      if (st == ST_REFINE && pass > 0 && suf - part < need && suf >= need) {
        uint32_t above = suf - part, cnt = 0;
        int bstar = (RBINS / TPV) * sub;
        for (int bin = (RBINS / TPV) * sub + RBINS / TPV - 1; bin >= (RBINS / TPV) * sub; --bin) {
          const uint32_t c = hist[v * HW + bin];
          if (above + c >= need) {
            bstar = bin;
            cnt = c;
            break;
          }
          above += c;
        }
        const u64 nlo = s_lo[v] + ((u64)bstar << s_shift[v]);
        const u64 top = nlo + (1ull << s_shift[v]);
        const u64 nhi = top < s_hi[v] ? top : s_hi[v];
        s_need[v] = (int)(need - above);
        s_lo[v] = nlo;
        s_hi[v] = nhi;
        if (cnt <= (uint32_t)CAP) {
          s_state[v] = ST_RCOLLECT;
        } else {
          const int bl = 64 - __clzll(nhi - nlo - 1);
          s_shift[v] = bl > 8 ? bl - 8 : 0;
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      int busy = 0;
      for (int v = 0; v < VT; ++v) busy |= (s_state[v] == ST_REFINE || s_state[v] == ST_RCOLLECT);
      // every refinement narrows the key range by >= 2^7 and K has 47 bits: a vector needs at
      // most 7 refinement sweeps and one collect sweep; the bound only guards the loop
      s_busy = busy && pass < 10;
    }
    for (int i = tid; i < VT * HW; i += THREADS) hist[i] = 0u;
    if (tid < VT) {
      s_above[tid] = s_state[tid] == ST_RCOLLECT ? 0 : s_above[tid];
      s_bcnt[tid] = 0;
    }
    __syncthreads();
    if (!s_busy) break;
    {
      LaneState ls{};
      ls.state = s_state[col];
      ls.active = ls.state == ST_REFINE || ls.state == ST_RCOLLECT;
      ls.lo = s_lo[col];
      ls.hi = s_hi[col];
      ls.shift = s_shift[col];
      sweep<DT, D, PASS_GENERIC>(dict_atoms, N, n, wave, col, h, b, ls, sh, pidx, psig);
    }
    __syncthreads();
  }
}

#define FADKV_SCORE_INST(DT, D)                                                                   \
  template __global__ void score_topn_kernel<DT, D>(const uint8_t *, const uint8_t *, int, int,  \
                                                    int, int, uint16_t *, float *, uint8_t *);
FADKV_SCORE_INST(DT_F32, 64)
FADKV_SCORE_INST(DT_F32, 128)
FADKV_SCORE_INST(DT_F16, 64)
FADKV_SCORE_INST(DT_F16, 128)
FADKV_SCORE_INST(DT_BF16, 64)
FADKV_SCORE_INST(DT_BF16, 128)

hipError_t launch_score_topn(int dtype, int d, const void *atoms, const void *X, int num_dicts,
                             int N, int M, int n, uint16_t *pool_idx, float *pool_sig,
                             uint8_t *vstat, hipStream_t stream) {
  const int nvb = (M + VT - 1) / VT;
  dim3 grid((unsigned)(8 * ((num_dicts + 7) / 8) * nvb)), block(THREADS);
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
#define L(DT, D)                                                                              \
  hipLaunchKernelGGL((score_topn_kernel<DT, D>), grid, block, 0, stream, A, Xb, num_dicts, N, M, \
                     n, pool_idx, pool_sig, vstat)
  if (dtype == DT_F32) { if (d == 64) L(DT_F32, 64); else L(DT_F32, 128); }
  else if (dtype == DT_F16) { if (d == 64) L(DT_F16, 64); else L(DT_F16, 128); }
  else { if (d == 64) L(DT_BF16, 64); else L(DT_BF16, 128); }
#undef L
  return hipGetLastError();
}

}  // namespace fadkv
