// Screening scores and exact Top-n candidate pool (FAD-KV abstract and Figure 1: one pass of
// dictionary correlations, then a one-shot Top-n pool by |score|, ties to the lowest index).
//
// One workgroup = 8 waves (4 for 512-byte rows) = one dictionary x 32 vectors.  The 32 vectors are the B operand of
// v_mfma_f32_32x32x{16,2}: they stay in registers for the whole dictionary sweep.  Each wave
// streams its own 32-atom tiles (A operand) straight from global memory/L2, prefetching the
// next tile while the current one is scored; a tile's 32x32 fp32 scores land in 16
// accumulators per lane, all belonging to the lane's vector (column lane % 32), so every score
// is handled by the lane that owns its vector.  Workgroups are numbered so that all
// workgroups of one dictionary land on the same XCD (dispatch is round-robin over the 8 XCDs),
// which keeps that dictionary in one L2.
//
// Selection is an exact radix select on the 47-bit key K = (bits(|score|) << 16) |
// (0xFFFF - atom): larger K = larger |score|, then lower index, and every K is unique.
//   pass 1 (level 0): histogram of |score| over 256 bins of 1/16 octave below ~||x||;
//   the bin holding the n-th largest key becomes the range [lo, hi);
//   if that bin holds more than CAP keys, further passes histogram the range uniformly;
//   final pass: keys >= hi go straight to the pool, keys in [lo, hi) go to an LDS buffer from
//   which the `need` largest are taken.
// Every pass recomputes the scores with the MFMA (bit-identical), so scores never leave chip.
#include "common.h"
#include "kernels.h"

namespace fadkv {

namespace {

constexpr int VT = 32;        // vectors per workgroup (one MFMA column block)
constexpr int BINS = 256;
constexpr int HSTRIDE = BINS + 1;   // padded histogram row: spreads vectors over LDS banks
constexpr int CAP = 64;             // boundary-bin capacity per vector

enum { MODE_HIST = 0, MODE_COLLECT = 1, MODE_DONE = 2 };

typedef unsigned long long u64;

template <int DT, int D> struct Geo {
  static constexpr int ROWB = D * Elem<DT>::bytes;   // bytes per row
  static constexpr int HALFB = ROWB / 2;             // bytes per lane (half a row)
  static constexpr int U4 = HALFB / 16;              // 16-byte chunks per lane fragment
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int GLD = 32 * CPR / 64;          // coalesced loads per lane per 32-row tile
  static constexpr int WAVES = CPR <= 16 ? 8 : 4;    // the per-wave stages must fit in LDS
  static constexpr int THREADS = WAVES * 64;
  static constexpr int STAGE_U4 = WAVES * 32 * (CPR + 1);
  static constexpr int TPV = THREADS / VT;           // threads per vector in the histogram scan
  static constexpr int BPT = BINS / TPV;             // bins per scanning thread
  static_assert(TPV <= 64 && (TPV & (TPV - 1)) == 0, "scan group must fit one wave");
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

// 32 rows starting at row0, coalesced: instruction i covers rows row0 + i*(64/CPR) + lane/CPR,
// chunk lane % CPR of each (rows >= N read as zeros)
template <int CPR, int GLD>
__device__ __forceinline__ void load_rows(uint4 (&g)[GLD], const uint8_t *base, int row0, int N,
                                          int rowb, int lane) {
#pragma unroll
  for (int i = 0; i < GLD; ++i) {
    const int row = row0 + i * (64 / CPR) + lane / CPR;
    g[i] = row < N ? reinterpret_cast<const uint4 *>(base + (size_t)row * rowb)[lane % CPR]
                   : make_uint4(0, 0, 0, 0);
  }
}
template <int CPR, int GLD>
__device__ __forceinline__ void store_stage(uint4 *stage, const uint4 (&g)[GLD], int lane) {
#pragma unroll
  for (int i = 0; i < GLD; ++i) stage[(i * (64 / CPR) + lane / CPR) * (CPR + 1) + lane % CPR] = g[i];
}

__device__ __forceinline__ u64 comp_key(uint32_t key31, int atom) {
  return ((u64)key31 << 16) | (u64)(0xFFFFu - (uint32_t)atom);
}

}  // namespace

template <int DT, int D>
__global__ __launch_bounds__(512) void score_topn_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int num_dicts, int N, int M,
    int n, uint16_t *__restrict__ pool_idx, float *__restrict__ pool_sig,
    uint8_t *__restrict__ vstat) {
  using G = Geo<DT, D>;
  __shared__ uint32_t hist[VT * HSTRIDE];
  __shared__ float bsig[VT * CAP];
  __shared__ int bidx[VT * CAP];
  __shared__ u64 s_lo[VT], s_hi[VT];
  __shared__ int s_mode[VT], s_need[VT], s_base[VT], s_shift[VT], s_above[VT], s_bcnt[VT];
  __shared__ int s_busy;
  __shared__ uint4 s_tile[G::STAGE_U4];

  // workgroup i runs on XCD i % 8; its r-th workgroup takes dictionary x + 8 * (r / B)
  const int nvb = (M + VT - 1) / VT;
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  const int dict = xcd + 8 * (r / nvb);
  if (dict >= num_dicts) return;
  const int v0 = (r % nvb) * VT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const uint8_t *dict_atoms = atoms + (size_t)dict * N * G::ROWB;
  const size_t vbase = (size_t)dict * M + v0;

  if (tid < VT) {
    int mode = MODE_DONE;
    if (v0 + tid < M) {
      const uint8_t *xr = X + (vbase + tid) * G::ROWB;
      float ss = 0.f;
      bool fin = true;
      for (int i = 0; i < D; ++i) {
        float f = elem_f<DT>(xr, i);
        fin = fin && __builtin_isfinite(f);
        ss += f * f;
      }
      uint8_t st = !fin ? VS_NONFINITE : (ss == 0.f ? VS_ZERO : VS_NORMAL);
      vstat[vbase + tid] = st;
      if (st == VS_NORMAL) {
        mode = MODE_HIST;
        // bin 246 holds |score| ~ ||x||; 246 bins of 1/16 octave below, 9 above
        s_base[tid] = (int)(__float_as_uint(sqrtf(ss)) >> 19) - 246;
      }
    }
    s_mode[tid] = mode;
    s_shift[tid] = -1;
    s_lo[tid] = 0;
    s_hi[tid] = 1ull << 47;
    s_need[tid] = n;
    s_above[tid] = 0;
    s_bcnt[tid] = 0;
  }

  uint4 b[G::U4];
  {
    const bool ok = v0 + col < M;
    const uint4 *src = reinterpret_cast<const uint4 *>(X + (vbase + col) * G::ROWB + h * G::HALFB);
#pragma unroll
    for (int i = 0; i < G::U4; ++i) b[i] = ok ? src[i] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int ntiles = (N + 31) / 32;
  // Each refinement level narrows the key range by >= 2^7 and K has 47 bits, so a vector needs
  // at most 1 + 7 histogram passes and one collect pass; the bound only guards the loop.
  for (int pass = 0;; ++pass) {
    if (tid == 0) {
      int busy = 0;
      for (int v = 0; v < VT; ++v) busy |= (s_mode[v] != MODE_DONE);
      s_busy = busy && pass < 12;
    }
    for (int i = tid; i < VT * HSTRIDE; i += G::THREADS) hist[i] = 0u;
    __syncthreads();
    if (!s_busy) break;

    const int mode = s_mode[col];
    const u64 lo = s_lo[col], hi = s_hi[col];
    const int base = s_base[col], shift = s_shift[col];
    uint16_t *pidx = pool_idx + (vbase + col) * (size_t)n;
    float *psig = pool_sig + (vbase + col) * (size_t)n;

    // Atom tiles reach the MFMA through a per-wave LDS stage: whole rows are read from global
    // memory with coalesced 16-byte loads (CPR lanes per row), the next tile's load is in flight
    // while the current tile is scored, and each lane then reads its MFMA fragment (half of row
    // lane % 32) from the stage.
    uint4 *stage = s_tile + wave * (32 * (G::CPR + 1));
    uint4 g[G::GLD];
    if (wave < ntiles) {
      load_rows<G::CPR, G::GLD>(g, dict_atoms, wave * 32, N, G::ROWB, lane);
      store_stage<G::CPR, G::GLD>(stage, g, lane);
    }
    for (int t = wave; t < ntiles; t += G::WAVES) {
      uint4 a[G::U4];
#pragma unroll
      for (int i = 0; i < G::U4; ++i) a[i] = stage[col * (G::CPR + 1) + h * G::U4 + i];
      const bool more = t + G::WAVES < ntiles;
      if (more) load_rows<G::CPR, G::GLD>(g, dict_atoms, (t + G::WAVES) * 32, N, G::ROWB, lane);
      const float16_t acc = tile_scores<DT, D>(a, b);
      if (more) store_stage<G::CPR, G::GLD>(stage, g, lane);
      if (mode == MODE_DONE) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int atom = t * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (atom >= N) continue;
        const float sc = acc[r];
        const uint32_t key = __float_as_uint(sc) & 0x7fffffffu;
        if (mode == MODE_HIST) {
          int bin;
          if (shift < 0) {
            bin = (int)(key >> 19) - base;
            bin = bin < 0 ? 0 : (bin > BINS - 1 ? BINS - 1 : bin);
          } else {
            const u64 K = comp_key(key, atom);
            if (K < lo || K >= hi) continue;
            bin = (int)((K - lo) >> shift);
          }
          atomicAdd(&hist[col * HSTRIDE + bin], 1u);
        } else {
          const u64 K = comp_key(key, atom);
          if (K >= hi) {
            const int pos = atomicAdd(&s_above[col], 1);
            if (pos < n) {
              pidx[pos] = (uint16_t)atom;
              psig[pos] = sc;
            }
          } else if (K >= lo) {
            const int pos = atomicAdd(&s_bcnt[col], 1);
            if (pos < CAP) {
              bsig[col * CAP + pos] = sc;
              bidx[col * CAP + pos] = atom;
            }
          }
        }
      }
    }
    __syncthreads();

    // vectors that collected this pass: take the `need` largest keys of the boundary bin
    for (int slot = tid; slot < VT * CAP; slot += G::THREADS) {
      const int v = slot / CAP, e = slot % CAP;
      const int cnt = s_bcnt[v] < CAP ? s_bcnt[v] : CAP;
      if (s_mode[v] != MODE_COLLECT || e >= cnt) continue;
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
      // TPV threads per vector: thread `sub` sums bins [BPT sub, BPT sub + BPT); a suffix sum
      // over the partial sums locates the bin holding the need-th largest key
      const int v = tid / G::TPV, sub = tid % G::TPV;
      const int mode_v = s_mode[v];
      uint32_t part = 0;
      if (mode_v == MODE_HIST) {
#pragma unroll
        for (int q = 0; q < G::BPT; ++q) part += hist[v * HSTRIDE + G::BPT * sub + q];
      }
      uint32_t suf = part;   // sum over sub' >= sub
#pragma unroll
      for (int o = 1; o < G::TPV; o <<= 1) {
        const uint32_t other = __shfl_down(suf, o, G::TPV);
        if (sub + o < G::TPV) suf += other;
      }
      const uint32_t above_grp = suf - part;   // keys in bins above this thread's 8 bins
      const int need = s_need[v];
      if (mode_v == MODE_COLLECT) {
        if (sub == 0) s_mode[v] = MODE_DONE;
      } else if (mode_v == MODE_HIST && above_grp < (uint32_t)need && suf >= (uint32_t)need) {
        uint32_t above = above_grp;
        int bstar = G::BPT * sub;
        for (int bin = G::BPT * sub + G::BPT - 1; bin >= G::BPT * sub; --bin) {
          const uint32_t c = hist[v * HSTRIDE + bin];
          if (above + c >= (uint32_t)need) {
            bstar = bin;
            break;
          }
          above += c;
        }
        const uint32_t cnt = hist[v * HSTRIDE + bstar];
        u64 nlo, nhi;
        if (s_shift[v] < 0) {
          const long long bs = s_base[v] + bstar;
          long long lob = bstar == 0 ? 0 : bs << 19;
          long long hib = bstar == BINS - 1 ? (1ll << 31) : (bs + 1) << 19;
          lob = lob < 0 ? 0 : lob;
          hib = hib < 0 ? 0 : (hib > (1ll << 31) ? (1ll << 31) : hib);
          nlo = (u64)lob << 16;
          nhi = (u64)hib << 16;
        } else {
          nlo = s_lo[v] + ((u64)bstar << s_shift[v]);
          const u64 top = nlo + (1ull << s_shift[v]);
          nhi = top < s_hi[v] ? top : s_hi[v];
        }
        s_need[v] = need - (int)above;
        s_lo[v] = nlo;
        s_hi[v] = nhi;
        if (cnt <= (uint32_t)CAP) {
          s_mode[v] = MODE_COLLECT;
          s_above[v] = 0;
          s_bcnt[v] = 0;
        } else {
          const u64 width = nhi - nlo;
          const int bl = 64 - __clzll(width - 1);
          s_shift[v] = bl > 8 ? bl - 8 : 0;
        }
      }
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
  dim3 grid((unsigned)(8 * ((num_dicts + 7) / 8) * nvb));
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
#define L(DT, D) \
  hipLaunchKernelGGL((score_topn_kernel<DT, D>), grid, dim3(Geo<DT, D>::THREADS), 0, stream, A, Xb, num_dicts, N, M, n, pool_idx, pool_sig, vstat)
  if (dtype == DT_F32) { if (d == 64) L(DT_F32, 64); else L(DT_F32, 128); }
  else if (dtype == DT_F16) { if (d == 64) L(DT_F16, 64); else L(DT_F16, 128); }
  else { if (d == 64) L(DT_BF16, 64); else L(DT_BF16, 128); }
#undef L
  return hipGetLastError();
}

}  // namespace fadkv
