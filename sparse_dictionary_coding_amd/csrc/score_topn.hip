// Screening scores and exact Top-n candidate pool (FAD-KV abstract and Figure 1: one pass of
// dictionary correlations, then a one-shot Top-n pool by |score|, ties to the lowest index).
//
// One workgroup = 8 waves = one dictionary x 32 vectors.  The 32 vectors are the B operands of
// v_mfma_f32_16x16x32 (two blocks of 16 vectors) and stay in registers for the whole sweep.
// Each wave streams its own 16-atom tiles.  A tile is copied global -> LDS by direct-to-LDS
// loads whose lanes read the rows contiguously (one load moves 1 KB, four lanes a 64-byte
// segment), then every lane reads its MFMA fragment (row lane % 16, 16-byte chunk
// 4 i + lane / 16) back from the wave's stage.  The stage keeps chunk c of row r at position
// c ^ swz(r), so the 16 rows of a fragment read fall in distinct LDS banks.  A tile's 16x16
// scores per block land as 4 accumulators per lane: vector lane % 16 of the block, atoms
// 4 (lane / 16) + e.  Workgroups are numbered so that all workgroups of one dictionary run on
// the same XCD (dispatch is round-robin over the 8 XCDs).
//
// Selection is an exact radix select on the 47-bit key K = (bits(|score|) << 16) |
// (0xFFFF - atom): larger K = larger |score|, then lower index, and every K is unique.
//   sweep 1: histogram of |score| in 256 bins of 1/32 octave below ~1.5 ||x||; the bin
//            holding the n-th largest key is the boundary;
//   sweep 2: keys above the boundary bin go straight to the pool, keys inside it go to an LDS
//            buffer of CAP entries from which the `need` largest keys are taken.
// A vector whose boundary bin holds more than CAP keys is refined by further sweeps that
// histogram its key range uniformly (256 bins each) until the boundary bin fits.  Every sweep
// recomputes the scores with the MFMA (bit-identical), so scores never leave the chip.  Each
// vector owns one LDS region that holds its histogram or, while it collects, its boundary
// buffer (a vector is in one state at a time).
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace fadkv {

namespace {

using namespace tile;

constexpr int VT = 32;           // vectors per workgroup (two MFMA column blocks)
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int RB = 256;          // bins of every histogram level
constexpr int CAP = 128;         // boundary-buffer capacity per vector (scores, then atoms)
constexpr int REGW = RB + 1;     // words per vector region: RB bins + a discard word
constexpr int DISCARD = RB;
constexpr int TPV = THREADS / VT;    // threads per vector in the histogram scans (16)
constexpr int SHIFT0 = 18;       // key >> 18 = 8 exponent bits + 5 mantissa bits
constexpr int TOP0 = 237;        // level-0 bin of |score| ~ ||x|| is TOP0; 18 bins (~1.5x) above
constexpr int QCAP = 128;        // per-wave hit queue of the collect sweep (a ring)

enum { ST_IDLE = 0, ST_HIST0, ST_COLLECT, ST_REFINE, ST_RCOLLECT };
enum { PASS_HIST0 = 0, PASS_COLLECT = 1, PASS_GENERIC = 2 };

typedef unsigned long long u64;

__device__ __forceinline__ u64 comp_key(uint32_t key31, int atom) {
  return ((u64)key31 << 16) | (u64)(0xFFFFu - (uint32_t)atom);
}

struct VecState {           // one of the lane's two vectors during one sweep
  bool active;
  int state;
  int vi;                   // vector within the workgroup
  int base;                 // level-0: key >> 18 of bin 0
  int off;                  // level-0: region word of (key >> 18) is (key >> 18) + off
  uint32_t lo32, hi32;      // boundary bin in 31-bit key space (level 0); lo32 = 2^32 - 1: no hit
  u64 lo, hi;               // boundary range in composite-key space (refinement)
  int shift;
  uint16_t *pidx;
  float *psig;
};

struct Shared {
  uint32_t *reg;            // VT regions of REGW words
  int *above;
  int *bcnt;
  const uint32_t *hi32;     // per vector: lowest key above its boundary bin
  uint16_t *pidx0;          // pool rows of the workgroup's first vector
  float *psig0;
};

// A wave's collect-sweep hits wait in its LDS ring (score bits, atom | vector << 16) until 64
// are there; then every lane takes one, reserves its slot (pool or boundary buffer) with one
// LDS atomic and stores it.  head and len are wave-uniform.
struct HitQueue {
  uint2 *ring;
  int head, len;
};

__device__ __forceinline__ void flush_hits(int count, HitQueue &hq, int lane, int n,
                                           const Shared &sh) {
  if (lane < count) {
    const uint2 e = hq.ring[(hq.head + lane) & (QCAP - 1)];
    const int atom = (int)(e.y & 0xFFFFu), vi = (int)(e.y >> 16);
    const bool hi = (e.x & 0x7fffffffu) >= sh.hi32[vi];
    const int pos = atomicAdd(hi ? &sh.above[vi] : &sh.bcnt[vi], 1);
    if (hi) {
      if (pos < n) {
        sh.pidx0[(size_t)vi * n + pos] = (uint16_t)atom;
        sh.psig0[(size_t)vi * n + pos] = __uint_as_float(e.x);
      }
    } else if (pos < CAP) {
      uint32_t *reg = sh.reg + vi * REGW;
      reg[pos] = e.x;
      reg[CAP + pos] = (uint32_t)atom;
    }
  }
  hq.head = (hq.head + count) & (QCAP - 1);
  hq.len -= count;
}

template <int PASS, bool CHECK>
__device__ __forceinline__ void process(const float4_t &acc, int atom0, int N, int n,
                                        const VecState &vs, const Shared &sh) {
  uint32_t *reg = sh.reg + vs.vi * REGW;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int atom = atom0 + e;
    const float sc = acc[e];
    const uint32_t key = __float_as_uint(sc) & 0x7fffffffu;
    if constexpr (PASS == PASS_HIST0) {
      const int kc = min(max((int)(key >> SHIFT0), vs.base), vs.base + RB - 1);
      int w = kc + vs.off;
      if (CHECK && atom >= N) w = vs.vi * REGW + DISCARD;
      atomicAdd(&sh.reg[w], 1u);
    } else {
      if (CHECK && atom >= N) continue;
      const u64 K = comp_key(key, atom);
      if (vs.state == ST_REFINE) {
        if (K >= vs.lo && K < vs.hi) atomicAdd(&reg[(int)((K - vs.lo) >> vs.shift)], 1u);
      } else if (K >= vs.hi) {
        const int pos = atomicAdd(&sh.above[vs.vi], 1);
        if (pos < n) {
          vs.pidx[pos] = (uint16_t)atom;
          vs.psig[pos] = sc;
        }
      } else if (K >= vs.lo) {
        const int pos = atomicAdd(&sh.bcnt[vs.vi], 1);
        if (pos < CAP) {
          reg[pos] = __float_as_uint(sc);
          reg[CAP + pos] = (uint32_t)atom;
        }
      }
    }
  }
}

// Collect pass over one tile for both vectors.  Hits (|score| at or above the boundary bin)
// are rare, so each lane first gathers its eight hit flags into a mask and the wave then loops
// over the hits, one per lane and round (rounds = the largest hit count of a lane, not eight),
// appending them to the wave's hit queue.
template <bool CHECK>
__device__ __forceinline__ void collect_tile(const float4_t &acc0, const float4_t &acc1, int atom0,
                                             int N, int n, const VecState (&vs)[2],
                                             const Shared &sh, HitQueue &hq, int lane) {
  const float v[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const VecState &q = vs[b >> 2];
    const uint32_t key = __float_as_uint(v[b]) & 0x7fffffffu;
    const bool ok = !CHECK || atom0 + (b & 3) < N;
    m |= (ok && key >= q.lo32) ? 1u << b : 0u;
  }
  for (;;) {
    const u64 hm = __builtin_amdgcn_ballot_w64(m != 0);
    if (!hm) break;
    if (m) {
      const int b = __builtin_ctz(m);
      m &= m - 1;
      // v[b] by a select tree on the bits of b (no indexed register access)
      const bool b0 = b & 1, b1 = b & 2, b2 = b & 4;
      const float c0 = b1 ? (b0 ? v[3] : v[2]) : (b0 ? v[1] : v[0]);
      const float c1 = b1 ? (b0 ? v[7] : v[6]) : (b0 ? v[5] : v[4]);
      const float sc = b2 ? c1 : c0;
      const int vi = b2 ? vs[1].vi : vs[0].vi;
      const int atom = atom0 + (b & 3);
      const int r = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hm >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)hm, 0u));
      hq.ring[(hq.head + hq.len + r) & (QCAP - 1)] =
          make_uint2(__float_as_uint(sc), (uint32_t)atom | ((uint32_t)vi << 16));
    }
    hq.len += __popcll(hm);          // <= 63 before the round, so <= 127 < QCAP after it
    if (hq.len >= 64) flush_hits(64, hq, lane, n, sh);
  }
}

// One sweep over the dictionary; PASS selects what every score of an active vector does.
// Wave w takes tiles w, w + 8, ...; REV runs them from the last one down, so that a sweep
// that follows another starts on the tiles the previous one left in L2.
template <int DT, int D, int PASS, bool REV = false>
__device__ __forceinline__ void sweep(const uint8_t *dict_atoms, int N, int n, int wave, int lane,
                                      const uint4 (&b)[2][Geo<DT, D>::CH], const VecState (&vs)[2],
                                      const Shared &sh, const uint4 *stage, uint32_t stage_lds,
                                      uint2 *ring) {
  using G = Geo<DT, D>;
  const int ntiles = (N + 15) / 16;
  const int r = lane % 16, g = lane / 16;
  uint32_t off[G::LOADS];
  tile_offsets<DT, D>(lane, off);
  if (wave >= ntiles) return;
  const int tlast = wave + (ntiles - 1 - wave) / WAVES * WAVES;
  const int tfirst = REV ? tlast : wave, step = REV ? -WAVES : WAVES;
  HitQueue hq{ring, 0, 0};
  issue_tile<DT, D>(dict_atoms, N, tfirst, lane, off, stage_lds);
  for (int t = tfirst; REV ? t >= 0 : t < ntiles; t += step) {
    wait_vmem();   // the tile is in the stage
    uint4 a[G::CH];
#pragma unroll
    for (int i = 0; i < G::CH; ++i) a[i] = stage[r * G::CPR + ((4 * i + g) ^ swz<G::CPR>(r))];
    wait_lds();    // fragments in registers: the stage may be overwritten
    if (REV ? t - WAVES >= 0 : t + WAVES < ntiles)
      issue_tile<DT, D>(dict_atoms, N, t + step, lane, off, stage_lds);
    float4_t acc0, acc1;
    tile_scores<DT, D>(a, b, acc0, acc1);
    const int atom0 = t * 16 + 4 * g;
    const bool full = t * 16 + 16 <= N;
    if constexpr (PASS == PASS_COLLECT) {
      if (full) collect_tile<false>(acc0, acc1, atom0, N, n, vs, sh, hq, lane);
      else collect_tile<true>(acc0, acc1, atom0, N, n, vs, sh, hq, lane);
    } else if (full) {
      if (vs[0].active) process<PASS, false>(acc0, atom0, N, n, vs[0], sh);
      if (vs[1].active) process<PASS, false>(acc1, atom0, N, n, vs[1], sh);
    } else {
      if (vs[0].active) process<PASS, true>(acc0, atom0, N, n, vs[0], sh);
      if (vs[1].active) process<PASS, true>(acc1, atom0, N, n, vs[1], sh);
    }
  }
  if constexpr (PASS == PASS_COLLECT) {
    while (hq.len > 0) flush_hits(hq.len < 64 ? hq.len : 64, hq, lane, n, sh);
  }
}

}  // namespace

template <int DT, int D>
__global__ __launch_bounds__(THREADS, (DT == DT_F32 && D == 128) ? 1 : 4) void score_topn_kernel(
    const uint8_t *__restrict__ atoms, const uint8_t *__restrict__ X, int num_dicts, int N, int M,
    int n, uint16_t *__restrict__ pool_idx, float *__restrict__ pool_sig,
    uint8_t *__restrict__ vstat, unsigned base) {
  using G = Geo<DT, D>;
  __shared__ __attribute__((aligned(16))) uint4 s_stage[WAVES * G::STAGE];
  __shared__ uint32_t s_reg[VT * REGW];
  __shared__ u64 s_lo[VT], s_hi[VT];
  __shared__ uint32_t s_lo32[VT], s_hi32[VT];
  __shared__ int s_state[VT], s_need[VT], s_base[VT], s_shift[VT], s_above[VT], s_bcnt[VT];
  __shared__ int s_busy;
  __shared__ uint2 s_queue[WAVES * QCAP];

  // workgroup i runs on XCD i % 8; its r-th workgroup takes dictionary x + 8 * (r / B).
  // (32-bit arithmetic: fewer than 2^31 workgroups over all chunks; base is a multiple of 8,
  // so the XCD of workgroup bid is still bid % 8)
  const unsigned bid = base + blockIdx.x;
  const unsigned nvb = (unsigned)(((size_t)M + VT - 1) / VT);
  const int xcd = (int)(bid % 8u);
  const unsigned rr = bid / 8u;
  const int dict = xcd + 8 * (int)(rr / nvb);
  if (dict >= num_dicts) return;
  const int v0 = (int)(rr % nvb) * VT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t *dict_atoms = atoms + (size_t)dict * N * G::ROWB;
  const size_t vbase = (size_t)dict * M + v0;
  const Shared sh{s_reg, s_above, s_bcnt, s_hi32, pool_idx + vbase * (size_t)n,
                  pool_sig + vbase * (size_t)n};
  uint2 *ring = s_queue + wave * QCAP;
  uint4 *stage = s_stage + wave * G::STAGE;
  // LDS byte address of the stage (wave-uniform, for M0)
  const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)stage);

  if (tid < VT) {
    int state = ST_IDLE;
    if (v0 + tid < M) {
      const uint4 *xr = reinterpret_cast<const uint4 *>(X + (vbase + tid) * G::ROWB);
      float ss = 0.f;
      bool fin = true;
      for (int c = 0; c < G::CPR; ++c) {
        const uint4 q = xr[c];
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (DT == DT_F32) {
            const float f = __uint_as_float(w4[u]);
            fin = fin && __builtin_isfinite(f);
            ss = fmaf(f, f, ss);
          } else {
            const float f0 = lo_f<DT>(w4[u]), f1 = hi_f<DT>(w4[u]);
            fin = fin && __builtin_isfinite(f0) && __builtin_isfinite(f1);
            ss = fmaf(f0, f0, ss);
            ss = fmaf(f1, f1, ss);
          }
        }
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
  // B fragments: block k, step i holds chunk 4 i + lane / 16 of vector 16 k + lane % 16
  uint4 b[2][G::CH];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int v = 16 * k + lane % 16;
    const bool ok = v0 + v < M;
    const uint4 *src = reinterpret_cast<const uint4 *>(X + (vbase + (ok ? v : 0)) * G::ROWB);
#pragma unroll
    for (int i = 0; i < G::CH; ++i) b[k][i] = ok ? src[4 * i + lane / 16] : make_uint4(0, 0, 0, 0);
  }
  for (int i = tid; i < VT * REGW; i += THREADS) s_reg[i] = 0u;
  __syncthreads();

  VecState vs[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    vs[k] = VecState{};
    vs[k].vi = 16 * k + lane % 16;
    vs[k].pidx = pool_idx + (vbase + vs[k].vi) * (size_t)n;
    vs[k].psig = pool_sig + (vbase + vs[k].vi) * (size_t)n;
  }

  // ---- sweep 1: level-0 histogram -----------------------------------------------------------
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    vs[k].active = s_state[vs[k].vi] == ST_HIST0;
    vs[k].base = s_base[vs[k].vi];
    vs[k].off = vs[k].vi * REGW - vs[k].base;
  }
  sweep<DT, D, PASS_HIST0>(dict_atoms, N, n, wave, lane, b, vs, sh, stage, stage_lds, ring);
  __syncthreads();
  {
    // TPV threads per vector: thread `sub` covers bins [16 sub, 16 sub + 16); a suffix sum of
    // the per-thread counts locates the bin holding the n-th largest key
    const int v = tid / TPV, sub = tid % TPV;
    const bool on = s_state[v] == ST_HIST0;
    constexpr int BPT = RB / TPV;
    uint32_t part = 0;
    if (on) {
#pragma unroll
      for (int q = 0; q < BPT; ++q) part += s_reg[v * REGW + BPT * sub + q];
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
      int bstar = BPT * sub;
      for (int bin = BPT * sub + BPT - 1; bin >= BPT * sub; --bin) {
        const uint32_t c = s_reg[v * REGW + bin];
        if (above + c >= need) {
          bstar = bin;
          cnt = c;
          break;
        }
        above += c;
      }
      const long long bs = (long long)s_base[v] + bstar;
      long long lob = bstar == 0 ? 0 : bs << SHIFT0;
      long long hib = bstar == RB - 1 ? (1ll << 31) : (bs + 1) << SHIFT0;
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
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    vs[k].active = s_state[vs[k].vi] == ST_COLLECT;
    // a vector that does not collect gets a bound no 31-bit key reaches, so the collect pass
    // needs no per-slot activity test
    vs[k].lo32 = vs[k].active ? s_lo32[vs[k].vi] : 0xFFFFFFFFu;
    vs[k].hi32 = s_hi32[vs[k].vi];
  }
  sweep<DT, D, PASS_COLLECT, true>(dict_atoms, N, n, wave, lane, b, vs, sh, stage, stage_lds, ring);
  __syncthreads();

  // ---- resolve boundaries; refine the rest (rare) -------------------------------------------
  for (int pass = 0;; ++pass) {
    // vectors that collected this pass: take the `need` largest keys of the boundary buffer.
    // One wave per vector; lane e holds entries e and e + 64 in registers, and each entry's
    // rank (the number of larger keys; keys are unique) counts the keys broadcast lane by lane.
    for (int v = wave; v < VT; v += WAVES) {
      const int st = __builtin_amdgcn_readfirstlane(s_state[v]);
      if (st != ST_COLLECT && st != ST_RCOLLECT) continue;
      const int cnt = __builtin_amdgcn_readfirstlane(s_bcnt[v] < CAP ? s_bcnt[v] : CAP);
      const uint32_t *reg = s_reg + v * REGW;
      const int e0 = lane, e1 = lane + 64;
      const u64 K0 = e0 < cnt ? comp_key(reg[e0] & 0x7fffffffu, (int)reg[CAP + e0]) : 0ull;
      const u64 K1 = e1 < cnt ? comp_key(reg[e1] & 0x7fffffffu, (int)reg[CAP + e1]) : 0ull;
      int r0 = 0, r1 = 0;
      for (int q = 0; q < cnt; ++q) {
        const u64 src = q < 64 ? K0 : K1;
        const int ql = q & 63;
        const uint32_t qh = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(src >> 32), ql);
        const uint32_t ql32 = (uint32_t)__builtin_amdgcn_readlane((uint32_t)src, ql);
        const u64 Kq = ((u64)qh << 32) | (u64)ql32;
        r0 += Kq > K0;
        r1 += Kq > K1;
      }
      const int need = s_need[v];
      if (need <= n) {
        const size_t row = (vbase + v) * (size_t)n;
        if (e0 < cnt && r0 < need) {
          pool_idx[row + n - need + r0] = (uint16_t)reg[CAP + e0];
          pool_sig[row + n - need + r0] = __uint_as_float(reg[e0]);
        }
        if (e1 < cnt && r1 < need) {
          pool_idx[row + n - need + r1] = (uint16_t)reg[CAP + e1];
          pool_sig[row + n - need + r1] = __uint_as_float(reg[e1]);
        }
      }
    }
    __syncthreads();
    {
      // refinement finalize: TPV threads per vector over RB bins
      const int v = tid / TPV, sub = tid % TPV;
      const int st = s_state[v];
      constexpr int BPT = RB / TPV;
      uint32_t part = 0;
      if (st == ST_REFINE && pass > 0) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) part += s_reg[v * REGW + BPT * sub + q];
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
        int bstar = BPT * sub;
        for (int bin = BPT * sub + BPT - 1; bin >= BPT * sub; --bin) {
          const uint32_t c = s_reg[v * REGW + bin];
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
    for (int i = tid; i < VT * REGW; i += THREADS) s_reg[i] = 0u;
    if (tid < VT) {
      s_above[tid] = s_state[tid] == ST_RCOLLECT ? 0 : s_above[tid];
      s_bcnt[tid] = 0;
    }
    __syncthreads();
    if (!s_busy) break;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int v = vs[k].vi;
      vs[k].state = s_state[v];
      vs[k].active = vs[k].state == ST_REFINE || vs[k].state == ST_RCOLLECT;
      vs[k].lo = s_lo[v];
      vs[k].hi = s_hi[v];
      vs[k].shift = s_shift[v];
    }
    sweep<DT, D, PASS_GENERIC>(dict_atoms, N, n, wave, lane, b, vs, sh, stage, stage_lds, ring);
    __syncthreads();
  }
}

#define FADKV_SCORE_INST(DT, D)                                                                   \
  template __global__ void score_topn_kernel<DT, D>(const uint8_t *, const uint8_t *, int, int,  \
                                                    int, int, uint16_t *, float *, uint8_t *,    \
                                                    unsigned);
FADKV_SCORE_INST(DT_F32, 64)
FADKV_SCORE_INST(DT_F32, 128)
FADKV_SCORE_INST(DT_F16, 64)
FADKV_SCORE_INST(DT_F16, 128)
FADKV_SCORE_INST(DT_BF16, 64)
FADKV_SCORE_INST(DT_BF16, 128)

hipError_t launch_score_topn(int dtype, int d, const void *atoms, const void *X, int num_dicts,
                             int N, int M, int n, uint16_t *pool_idx, float *pool_sig,
                             uint8_t *vstat, hipStream_t stream) {
  const size_t nvb = ((size_t)M + VT - 1) / VT;
  // num_dicts * M < 2^31 vectors: fewer than 2^31 workgroups; launched in chunks of at most
  // kMaxBlocksPerLaunch (a multiple of 8, so every chunk keeps the XCD numbering)
  const size_t total = 8 * (((size_t)num_dicts + 7) / 8) * nvb;
  const uint8_t *A = static_cast<const uint8_t *>(atoms);
  const uint8_t *Xb = static_cast<const uint8_t *>(X);
  for (size_t b0 = 0; b0 < total; b0 += kMaxBlocksPerLaunch) {
    const size_t nb = total - b0 < kMaxBlocksPerLaunch ? total - b0 : kMaxBlocksPerLaunch;
    const dim3 grid((unsigned)nb), block(THREADS);
#define L(DT, D)                                                                              \
  hipLaunchKernelGGL((score_topn_kernel<DT, D>), grid, block, 0, stream, A, Xb, num_dicts, N, M, \
                     n, pool_idx, pool_sig, vstat, (unsigned)b0)
    if (dtype == DT_F32) { if (d == 64) L(DT_F32, 64); else L(DT_F32, 128); }
    else if (dtype == DT_F16) { if (d == 64) L(DT_F16, 64); else L(DT_F16, 128); }
    else { if (d == 64) L(DT_BF16, 64); else L(DT_BF16, 128); }
#undef L
  }
  return hipGetLastError();
}

}  // namespace fadkv
