// C ABI of libfadkv (declared in include/fadkv.h): argument checks on the host, workspace
// carving and kernel dispatch.  Nothing here allocates, synchronises or touches the GPU before
// every argument has been accepted.
#include "fadkv.h"

#include <math.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr int kMaxN = 65535;    // pool indices are stored as uint16
constexpr int kMaxPool = 512;   // one selection thread per pool entry
constexpr int kMaxS = 32;
constexpr int kMaxAttendN = 16384;   // a query's q . D_K^T row and atom weights live in LDS
// the attention kernels' grids: one 1024-thread workgroup per row, d threads per query output
constexpr int64_t kMaxAttendR = int64_t(1) << 22;
constexpr int64_t kMaxAttendRG = int64_t(1) << 24;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Layout {
  // encode
  size_t pool_idx, pool_sig, vstat, encode_end;
  // adapt
  size_t touched, rank, cand, ccount, adapt_end;
  int touched_stride;
  size_t total;
};

Layout layout(const fadkv_dict *dict, const fadkv_params *p, int64_t M) {
  Layout L{};
  const size_t G = (size_t)dict->num_dicts * (size_t)M;
  size_t o = 0;
  L.pool_idx = o; o = align_up(o + G * (size_t)p->n * sizeof(uint16_t));
  L.pool_sig = o; o = align_up(o + G * (size_t)p->n * sizeof(float));
  L.vstat = o;    o = align_up(o + G);
  L.encode_end = o;
  o = 0;
  L.touched_stride = (int)align_up((size_t)dict->N);
  L.touched = o; o = align_up(o + (size_t)dict->num_dicts * L.touched_stride);
  L.rank = o;    o = align_up(o + G * sizeof(int32_t));
  L.cand = o;    o = align_up(o + G * sizeof(int32_t));
  L.ccount = o;  o = align_up(o + (size_t)dict->num_dicts * sizeof(int32_t));
  L.adapt_end = o;
  L.total = L.encode_end > L.adapt_end ? L.encode_end : L.adapt_end;
  return L;
}

int check_dict(const fadkv_dict *dict) {
  if (!dict) return FADKV_ERR_ARG;
  if (dict->dtype != FADKV_F32 && dict->dtype != FADKV_F16 && dict->dtype != FADKV_BF16)
    return FADKV_ERR_DTYPE;
  if (dict->num_dicts < 1 || dict->N < 1 || dict->N > kMaxN) return FADKV_ERR_SHAPE;
  if (dict->d != 64 && dict->d != 128) return FADKV_ERR_SHAPE;
  if (!dict->atoms || !aligned(dict->atoms, 16)) return FADKV_ERR_ARG;
  return FADKV_OK;
}

int check_params(const fadkv_dict *dict, const fadkv_params *p) {
  if (!p) return FADKV_ERR_ARG;
  if (p->s < 1 || p->s > kMaxS || p->n < p->s || p->n > kMaxPool || p->n > dict->N)
    return FADKV_ERR_SHAPE;
  if (p->select != FADKV_SELECT_GM && p->select != FADKV_SELECT_PL) return FADKV_ERR_ARG;
  if (!(p->ridge_abs >= 0.f) || !(p->ridge_rel >= 0.f) || !isfinite(p->ridge_abs) ||
      !isfinite(p->ridge_rel))
    return FADKV_ERR_ARG;
  if (!(p->delta_key >= 0.f) || !(p->delta_value >= 0.f)) return FADKV_ERR_ARG;
  return FADKV_OK;
}

int check_M(const fadkv_dict *dict, int64_t M) {
  if (M < 0) return FADKV_ERR_ARG;
  if ((double)dict->num_dicts * (double)M >= 2147483648.0) return FADKV_ERR_SHAPE;
  return FADKV_OK;
}

int check_codes(const fadkv_codes *c) {
  if (!c || !c->idx || !c->coef || !c->relerr || !c->flags) return FADKV_ERR_ARG;
  if (!aligned(c->idx, 4) || !aligned(c->coef, 4) || !aligned(c->relerr, 4)) return FADKV_ERR_ARG;
  return FADKV_OK;
}

// q . D_K^T, then the atom weights, [R*G][N] fp32; then [ranges of 128 atoms][R*G][d] fp32
size_t attend_ws_bytes(const fadkv_dict *dict, int64_t R, int32_t G) {
  const size_t RG = (size_t)R * (size_t)G;
  const size_t ranges = ((size_t)dict->N + 127) / 128;
  return align_up(RG * (size_t)dict->N * sizeof(float) + ranges * RG * (size_t)dict->d * sizeof(float));
}

struct OmpLayout {
  size_t status, jstar, S, L, sig, R, total;
};

OmpLayout omp_layout(const fadkv_dict *dict, const fadkv_params *p, int64_t M) {
  OmpLayout L{};
  const size_t G = (size_t)dict->num_dicts * (size_t)M;
  const size_t s = (size_t)p->s;
  size_t o = 0;
  L.status = o; o = align_up(o + G);
  L.jstar = o;  o = align_up(o + G * sizeof(int32_t));
  L.S = o;      o = align_up(o + G * s * sizeof(int32_t));
  L.L = o;      o = align_up(o + G * s * s * sizeof(float));
  L.sig = o;    o = align_up(o + G * s * sizeof(float));
  L.R = o;      o = align_up(o + G * fadkv::omp_residual_row_bytes(dict->dtype, dict->d));
  L.total = o;
  return L;
}

// the support/coefficient stage of the chosen selection mode
hipError_t run_select(const fadkv_dict *dict, const fadkv_params *p, const void *X, int64_t M,
                      const uint16_t *pool_idx, const float *pool_sig, const uint8_t *vstat,
                      const fadkv_codes *out, hipStream_t stream) {
  if (p->select == FADKV_SELECT_PL)
    return fadkv::launch_select_pl(dict->dtype, dict->d, dict->atoms, X, dict->num_dicts, dict->N,
                                   (int)M, p->n, p->s, p->ridge_abs, p->ridge_rel, p->delta_key,
                                   p->delta_value, pool_idx, pool_sig, vstat, out->idx, out->coef,
                                   out->relerr, out->flags, stream);
  return fadkv::launch_select(dict->dtype, dict->d, dict->atoms, X, dict->num_dicts, dict->N,
                              (int)M, p->n, p->s, p->ridge_abs, p->ridge_rel, p->delta_key,
                              p->delta_value, pool_idx, pool_sig, vstat, out->idx, out->coef,
                              out->relerr, out->flags, stream);
}

// ---- static scratch of fadkv_encode_noalloc ---------------------------------------------------
// The array's name is only a host-side stand-in in host code: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address
// is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[FADKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once taken

int scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FADKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FADKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FADKV_OK;
}

#define FADKV_TRY(expr)        \
  do {                         \
    const int _st = (expr);    \
    if (_st != FADKV_OK) return _st; \
  } while (0)

}  // namespace

extern "C" {

int fadkv_abi_version(void) { return FADKV_ABI_VERSION; }

const char *fadkv_status_string(int status) {
  switch (status) {
    case FADKV_OK: return "ok";
    case FADKV_ERR_ARG: return "invalid argument (null or misaligned pointer, negative count or bad parameter)";
    case FADKV_ERR_DTYPE: return "unsupported dtype";
    case FADKV_ERR_SHAPE: return "shape outside the supported limits";
    case FADKV_ERR_WORKSPACE: return "workspace missing or too small";
    case FADKV_ERR_HIP: return "HIP runtime or kernel launch failure";
    case FADKV_ERR_SCRATCH:
      return "fadkv_encode_noalloc needs more than its static scratch (FADKV_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int fadkv_workspace_bytes(const fadkv_dict *dict, const fadkv_params *params, int64_t M,
                          size_t *bytes) {
  if (!bytes) return FADKV_ERR_ARG;
  if (!dict) return FADKV_ERR_ARG;
  if (dict->dtype != FADKV_F32 && dict->dtype != FADKV_F16 && dict->dtype != FADKV_BF16)
    return FADKV_ERR_DTYPE;
  if (dict->num_dicts < 1 || dict->N < 1 || dict->N > kMaxN || (dict->d != 64 && dict->d != 128))
    return FADKV_ERR_SHAPE;
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  *bytes = layout(dict, params, M).total;
  return FADKV_OK;
}

int fadkv_encode(const fadkv_dict *dict, const fadkv_params *params, const void *X, int64_t M,
                 const fadkv_codes *out, void *workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  FADKV_TRY(check_codes(out));
  if (M > 0 && (!X || !aligned(X, 16))) return FADKV_ERR_ARG;
  const Layout L = layout(dict, params, M);
  if (M > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < L.total))
    return FADKV_ERR_WORKSPACE;
  if (M == 0) return FADKV_OK;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  uint16_t *pool_idx = reinterpret_cast<uint16_t *>(ws + L.pool_idx);
  float *pool_sig = reinterpret_cast<float *>(ws + L.pool_sig);
  uint8_t *vstat = ws + L.vstat;
  if (fadkv::launch_score_topn(dict->dtype, dict->d, dict->atoms, X, dict->num_dicts, dict->N,
                               (int)M, params->n, pool_idx, pool_sig, vstat, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  if (run_select(dict, params, X, M, pool_idx, pool_sig, vstat, out, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_encode_noalloc(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                         int64_t M, const fadkv_codes *out, hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  FADKV_TRY(check_codes(out));
  if (M > 0 && (!X || !aligned(X, 16))) return FADKV_ERR_ARG;
  const Layout L = layout(dict, params, M);
  if (L.encode_end > FADKV_NOALLOC_SCRATCH_BYTES) return FADKV_ERR_SCRATCH;
  if (M == 0) return FADKV_OK;
  void *ptr = nullptr;
  FADKV_TRY(scratch_of_current_device(&ptr));
  uint8_t *ws = static_cast<uint8_t *>(ptr);
  uint16_t *pool_idx = reinterpret_cast<uint16_t *>(ws + L.pool_idx);
  float *pool_sig = reinterpret_cast<float *>(ws + L.pool_sig);
  uint8_t *vstat = ws + L.vstat;
  if (fadkv::launch_score_topn(dict->dtype, dict->d, dict->atoms, X, dict->num_dicts, dict->N,
                               (int)M, params->n, pool_idx, pool_sig, vstat, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  if (run_select(dict, params, X, M, pool_idx, pool_sig, vstat, out, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_screen(const fadkv_dict *dict, const fadkv_params *params, const void *X, int64_t M,
                 uint16_t *pool_idx, float *pool_score, uint8_t *vstatus, hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  if (M == 0) return FADKV_OK;
  if (!X || !aligned(X, 16)) return FADKV_ERR_ARG;
  if (!pool_idx || !pool_score || !vstatus || !aligned(pool_idx, 2) || !aligned(pool_score, 4))
    return FADKV_ERR_ARG;
  if (fadkv::launch_score_topn(dict->dtype, dict->d, dict->atoms, X, dict->num_dicts, dict->N,
                               (int)M, params->n, pool_idx, pool_score, vstatus, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_select_support(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                         int64_t M, const uint16_t *pool_idx, const float *pool_score,
                         const uint8_t *vstatus, const fadkv_codes *out, hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  FADKV_TRY(check_codes(out));
  if (M == 0) return FADKV_OK;
  if (!X || !aligned(X, 16)) return FADKV_ERR_ARG;
  if (!pool_idx || !pool_score || !vstatus || !aligned(pool_idx, 2) || !aligned(pool_score, 4))
    return FADKV_ERR_ARG;
  if (run_select(dict, params, X, M, pool_idx, pool_score, vstatus, out, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_adapt(const fadkv_dict *dict, const fadkv_params *params, const void *X, int64_t M,
                const fadkv_codes *codes, int32_t *replaced, void *workspace,
                size_t workspace_bytes, hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  FADKV_TRY(check_codes(codes));
  if (!dict->usage || !aligned(dict->usage, 4)) return FADKV_ERR_ARG;
  if (!replaced || !aligned(replaced, 4)) return FADKV_ERR_ARG;
  if (M > 0 && (!X || !aligned(X, 16))) return FADKV_ERR_ARG;
  const Layout L = layout(dict, params, M);
  if (M > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < L.total))
    return FADKV_ERR_WORKSPACE;
  if (M == 0) return FADKV_OK;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  if (fadkv::launch_adapt(dict->dtype, dict->d, dict->atoms, dict->usage, X, dict->num_dicts,
                          dict->N, (int)M, params->s, params->ridge_abs, params->ridge_rel,
                          params->tau_c, codes->idx, codes->coef, codes->relerr, codes->flags,
                          replaced, ws + L.touched, L.touched_stride,
                          reinterpret_cast<int32_t *>(ws + L.rank),
                          reinterpret_cast<int32_t *>(ws + L.cand),
                          reinterpret_cast<int32_t *>(ws + L.ccount), nullptr,
                          stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_omp_workspace_bytes(const fadkv_dict *dict, const fadkv_params *params, int64_t M,
                              size_t *bytes) {
  if (!bytes || !dict) return FADKV_ERR_ARG;
  if (dict->dtype != FADKV_F32 && dict->dtype != FADKV_F16 && dict->dtype != FADKV_BF16)
    return FADKV_ERR_DTYPE;
  if (dict->num_dicts < 1 || dict->N < 1 || dict->N > kMaxN || (dict->d != 64 && dict->d != 128))
    return FADKV_ERR_SHAPE;
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  *bytes = omp_layout(dict, params, M).total;
  return FADKV_OK;
}

int fadkv_encode_omp(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                     int64_t M, const fadkv_codes *out, void *workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  FADKV_TRY(check_codes(out));
  if (M > 0 && (!X || !aligned(X, 16))) return FADKV_ERR_ARG;
  const OmpLayout L = omp_layout(dict, params, M);
  if (M > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < L.total))
    return FADKV_ERR_WORKSPACE;
  if (M == 0) return FADKV_OK;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  fadkv::OmpArgs a{};
  a.atoms = dict->atoms;
  a.X = X;
  a.num_dicts = dict->num_dicts;
  a.N = dict->N;
  a.M = (int)M;
  a.s = params->s;
  a.ridge_abs = params->ridge_abs;
  a.ridge_rel = params->ridge_rel;
  a.delta_key = params->delta_key;
  a.delta_value = params->delta_value;
  a.status = ws + L.status;
  a.jstar = reinterpret_cast<int32_t *>(ws + L.jstar);
  a.S = reinterpret_cast<int32_t *>(ws + L.S);
  a.L = reinterpret_cast<float *>(ws + L.L);
  a.sig = reinterpret_cast<float *>(ws + L.sig);
  a.R = ws + L.R;
  a.idx = out->idx;
  a.coef = out->coef;
  a.relerr = out->relerr;
  a.flags = out->flags;
  if (fadkv::launch_omp(dict->dtype, dict->d, a, stream) != hipSuccess) return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_adapt_append(const fadkv_dict *dict, const fadkv_params *params, const void *X,
                       int64_t M, const fadkv_codes *codes, int32_t *replaced, int32_t *n_atoms,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_params(dict, params));
  FADKV_TRY(check_M(dict, M));
  FADKV_TRY(check_codes(codes));
  if (!dict->usage || !aligned(dict->usage, 4)) return FADKV_ERR_ARG;
  if (!replaced || !aligned(replaced, 4)) return FADKV_ERR_ARG;
  if (!n_atoms || !aligned(n_atoms, 4)) return FADKV_ERR_ARG;
  if (M > 0 && (!X || !aligned(X, 16))) return FADKV_ERR_ARG;
  const Layout L = layout(dict, params, M);
  if (M > 0 && (!workspace || !aligned(workspace, kAlign) || workspace_bytes < L.total))
    return FADKV_ERR_WORKSPACE;
  if (M == 0) return FADKV_OK;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  if (fadkv::launch_adapt(dict->dtype, dict->d, dict->atoms, dict->usage, X, dict->num_dicts,
                          dict->N, (int)M, params->s, params->ridge_abs, params->ridge_rel,
                          params->tau_c, codes->idx, codes->coef, codes->relerr, codes->flags,
                          replaced, ws + L.touched, L.touched_stride,
                          reinterpret_cast<int32_t *>(ws + L.rank),
                          reinterpret_cast<int32_t *>(ws + L.cand),
                          reinterpret_cast<int32_t *>(ws + L.ccount), n_atoms,
                          stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_reconstruct(const fadkv_dict *dict, const int32_t *idx, const float *coef, int32_t s,
                      int64_t M, void *X_hat, int32_t out_dtype, hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  FADKV_TRY(check_M(dict, M));
  if (s < 1 || s > kMaxS) return FADKV_ERR_SHAPE;
  if (out_dtype != FADKV_F32 && out_dtype != FADKV_F16 && out_dtype != FADKV_BF16)
    return FADKV_ERR_DTYPE;
  if (M == 0) return FADKV_OK;
  if (!idx || !coef || !X_hat || !aligned(idx, 4) || !aligned(coef, 4) || !aligned(X_hat, 16))
    return FADKV_ERR_ARG;
  if (fadkv::launch_reconstruct(dict->dtype, dict->d, dict->atoms, idx, coef, dict->num_dicts,
                                dict->N, (int)M, s, X_hat, out_dtype, stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

int fadkv_attend_workspace_bytes(const fadkv_dict *dict, int64_t R, int32_t G, size_t *bytes) {
  if (!bytes || !dict) return FADKV_ERR_ARG;
  if (dict->dtype != FADKV_F32 && dict->dtype != FADKV_F16 && dict->dtype != FADKV_BF16)
    return FADKV_ERR_DTYPE;
  if (dict->num_dicts < 2 || dict->N < 1 || dict->N > kMaxAttendN ||
      (dict->d != 64 && dict->d != 128))
    return FADKV_ERR_SHAPE;
  if (R < 0 || G < 1 || G > 64) return FADKV_ERR_SHAPE;
  if (R > kMaxAttendR || (double)R * (double)G > (double)kMaxAttendRG) return FADKV_ERR_SHAPE;
  *bytes = attend_ws_bytes(dict, R, G);
  return FADKV_OK;
}

int fadkv_attend(const fadkv_dict *dict, int32_t layer, int32_t s, const int32_t *k_idx,
                 const float *k_coef, const int32_t *v_idx, const float *v_coef,
                 const int32_t *lens, int64_t R, int32_t T, const void *q, int32_t G,
                 float scale, float *out, void *workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  FADKV_TRY(check_dict(dict));
  if (dict->N > kMaxAttendN) return FADKV_ERR_SHAPE;
  if (layer < 0 || 2 * (int64_t)layer + 1 >= dict->num_dicts) return FADKV_ERR_SHAPE;
  if (s < 1 || s > kMaxS || R < 0 || T < 0 || G < 1 || G > 64) return FADKV_ERR_SHAPE;
  if (R > kMaxAttendR || (double)R * (double)G > (double)kMaxAttendRG) return FADKV_ERR_SHAPE;
  if ((double)R * (double)T * (double)s >= 9.0e18) return FADKV_ERR_SHAPE;
  if (!isfinite(scale)) return FADKV_ERR_ARG;
  if (R == 0) return FADKV_OK;
  if (!lens || !q || !out || !aligned(lens, 4) || !aligned(q, 16) || !aligned(out, 4))
    return FADKV_ERR_ARG;
  if (T > 0 && (!k_idx || !k_coef || !v_idx || !v_coef || !aligned(k_idx, 4) ||
                !aligned(k_coef, 4) || !aligned(v_idx, 4) || !aligned(v_coef, 4)))
    return FADKV_ERR_ARG;
  const size_t need = attend_ws_bytes(dict, R, G);
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < need)
    return FADKV_ERR_WORKSPACE;
  const size_t esize = dict->dtype == FADKV_F32 ? 4 : 2;
  const size_t dict_bytes = (size_t)dict->N * (size_t)dict->d * esize;
  const uint8_t *atoms = static_cast<const uint8_t *>(dict->atoms);
  if (fadkv::launch_attend(dict->dtype, dict->d, atoms + (size_t)(2 * layer) * dict_bytes,
                           atoms + (size_t)(2 * layer + 1) * dict_bytes, dict->N, s, k_idx, k_coef,
                           v_idx, v_coef, lens, (int)R, T, q, G, scale, out,
                           static_cast<float *>(workspace), stream) != hipSuccess)
    return FADKV_ERR_HIP;
  return FADKV_OK;
}

}  // extern "C"
