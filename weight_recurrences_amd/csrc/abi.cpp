// C ABI of the library (declared in include/linattn.h): argument validation,
// workspace sizing and dispatch to the gfx950 kernels.  Every check runs on
// the host before anything is enqueued, so an invalid call leaves the device
// untouched and never calls into the HIP runtime.
#include <stdint.h>

#include <algorithm>
#include <initializer_list>

#include "linattn.h"
#include "kernels.hpp"

namespace {

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when hi == lo
  Span() = default;
  Span(const void* p, long long bytes) : lo((uintptr_t)p), hi((uintptr_t)p + (uintptr_t)(p ? bytes : 0)) {}
  bool empty() const { return hi <= lo; }
  bool overlaps(const Span& o) const { return !empty() && !o.empty() && lo < o.hi && o.lo < hi; }
  bool same(const Span& o) const { return lo == o.lo && hi == o.hi; }
};

bool dm_supported(int D, int M) { return (D == 32 || D == 64) && (M == 32 || M == 64); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize(int dtype) { return dtype == LINATTN_BF16 ? 2 : 4; }

// Shape checks shared by the sequence entry points.  Sizes fit int64 element
// counts and the kernels' 32-bit grid and index arithmetic.
int check_shape(int B, int H, int N, int D, int M, int dtype) {
  if (dtype != LINATTN_F32 && dtype != LINATTN_BF16) return LINATTN_ERR_DTYPE;
  if (B < 0 || H < 0 || N < 0 || D <= 0 || M <= 0) return LINATTN_ERR_SHAPE;
  if (!dm_supported(D, M)) return LINATTN_ERR_UNSUPPORTED;
  // Token indices and block counts are 32-bit in the kernels and their launch
  // arithmetic (N + block - 1 included): at most 2^30 tokens per sequence.
  if (N > (1 << 30)) return LINATTN_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 30)) return LINATTN_ERR_SHAPE;
  const long long rows = BH * N;
  if (N > 0 && rows / N != BH) return LINATTN_ERR_SHAPE;
  if (rows > (1LL << 46) / 64) return LINATTN_ERR_SHAPE;  // bytes of q stay far below 2^63
  if (BH > 0 && N > 0) {
    const int tb = la::causal_block_tokens((int)BH, N);
    const long long nblk = ((long long)N + tb - 1) / tb;
    if (nblk * BH > (long long)INT32_MAX) return LINATTN_ERR_SHAPE;
  }
  return LINATTN_OK;
}

int check_align(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LINATTN_ERR_ALIGN;
  return LINATTN_OK;
}

// beta is read one element at a time: it needs only the alignment of its element.
int check_align_elem(const void* p, int es) {
  return (p && ((uintptr_t)p % (uintptr_t)es) != 0) ? LINATTN_ERR_ALIGN : LINATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP; }

}  // namespace

extern "C" {

size_t linattn_causal_workspace_bytes(int B, int H, int N, int D, int M, int dtype) {
  if (check_shape(B, H, N, D, M, dtype) != LINATTN_OK) return 0;
  return la::causal_ws_bytes(B * H, N, D, M, dtype == LINATTN_BF16);
}

size_t linattn_causal_bwd_workspace_bytes(int B, int H, int N, int D, int M, int dtype) {
  if (check_shape(B, H, N, D, M, dtype) != LINATTN_OK) return 0;
  return la::causal_bwd_ws_bytes(B * H, N, D, M);
}

int linattn_causal_bwd(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk, void* dv,
                       int B, int H, int N, int D, int M, int dtype, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(B, H, N, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH * N == 0) return LINATTN_OK;
  if (!q || !k || !v || !dO || !dq || !dk || !dv) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, dO, dq, dk, dv, ws}))) return st;
  const size_t need = la::causal_bwd_ws_bytes((int)BH, N, D, M);
  if (need > 0 && (!ws || ws_bytes < need)) return LINATTN_ERR_WORKSPACE;
  const long long nq = BH * N * D * es, nv = BH * N * M * es;
  const Span sq(q, nq), sk(k, nq), sv(v, nv), sg(dO, nv), sdq(dq, nq), sdk(dk, nq), sdv(dv, nv), sws(ws, (long long)need);
  for (const Span& out : {sdq, sdk, sdv})
    for (const Span& x : {sq, sk, sv, sg, sws})
      if (out.overlaps(x)) return LINATTN_ERR_ALIAS;
  if (sdq.overlaps(sdk) || sdq.overlaps(sdv) || sdk.overlaps(sdv)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sg})
    if (sws.overlaps(x)) return LINATTN_ERR_ALIAS;
  return hip_status(la::launch_causal_bwd(q, k, v, dO, dq, dk, dv, (int)BH, N, D, M, dtype == LINATTN_BF16, ws,
                                          (hipStream_t)stream));
}

size_t linattn_noncausal_workspace_bytes(int B, int H, int N, int D, int M, int dtype) {
  if (check_shape(B, H, N, D, M, dtype) != LINATTN_OK) return 0;
  return la::noncausal_ws_bytes(B * H, N, D, M, dtype == LINATTN_BF16);
}

int linattn_causal_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D, int M,
                       int dtype, const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                       size_t ws_bytes, void* stream) {
  int st = check_shape(B, H, N, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  const long long nq = BH * N * D * es, nv = BH * N * M * es;
  if ((S0 == nullptr) != (z0 == nullptr)) return LINATTN_ERR_NULL;
  if ((S_out == nullptr) != (z_out == nullptr)) return LINATTN_ERR_NULL;
  if (BH * N > 0 && (!q || !k || !v)) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, S0, z0, S_out, z_out, ws}))) return st;
  const size_t need = la::causal_ws_bytes((int)BH, N, D, M, dtype == LINATTN_BF16);
  const bool uses_ws = need > 0;
  if (uses_ws && (!ws || ws_bytes < need)) return LINATTN_ERR_WORKSPACE;

  const Span sq(q, nq), sk(k, nq), sv(v, nv), so(o, o ? nv : 0);
  const Span sS0(S0, BH * D * M * 4), sz0(z0, BH * D * 4), sSo(S_out, BH * D * M * 4), szo(z_out, BH * D * 4);
  const Span sws(ws, uses_ws ? (long long)need : 0);
  for (const Span& x : {sq, sk, sv, sS0, sz0, sSo, szo, sws})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& out : {sSo, szo})
    for (const Span& x : {sq, sk, sv, sws})
      if (out.overlaps(x)) return LINATTN_ERR_ALIAS;
  if (sSo.overlaps(szo)) return LINATTN_ERR_ALIAS;
  if ((sSo.overlaps(sS0) && !sSo.same(sS0)) || (szo.overlaps(sz0) && !szo.same(sz0))) return LINATTN_ERR_ALIAS;
  if (sSo.overlaps(sz0) || szo.overlaps(sS0)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sS0, sz0})
    if (sws.overlaps(x)) return LINATTN_ERR_ALIAS;

  if (BH == 0) return LINATTN_OK;
  if (N == 0 && !S_out) return LINATTN_OK;
  return hip_status(la::launch_causal(q, k, v, o, (int)BH, N, D, M, dtype == LINATTN_BF16, S0, z0, S_out, z_out,
                                      uses_ws ? ws : nullptr, (hipStream_t)stream));
}

int linattn_noncausal_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D, int M,
                          int dtype, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(B, H, N, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH * N == 0) return LINATTN_OK;
  const long long nq = BH * N * D * es, nv = BH * N * M * es;
  if (!q || !k || !v || !o) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, ws}))) return st;
  const size_t need = la::noncausal_ws_bytes((int)BH, N, D, M, dtype == LINATTN_BF16);
  if (!ws || ws_bytes < need) return LINATTN_ERR_WORKSPACE;
  const Span sq(q, nq), sk(k, nq), sv(v, nv), so(o, nv), sws(ws, (long long)need);
  for (const Span& x : {sq, sk, sv, sws})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv})
    if (sws.overlaps(x)) return LINATTN_ERR_ALIAS;
  return hip_status(
      la::launch_noncausal(q, k, v, o, (int)BH, N, D, M, dtype == LINATTN_BF16, ws, (hipStream_t)stream));
}

int linattn_noncausal_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D,
                                  int M, int dtype, void* stream) {
  int st = check_shape(B, H, N, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH * N == 0) return LINATTN_OK;
  if (!q || !k || !v || !o) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o}))) return st;
  // The same kernels and partition as linattn_noncausal_fwd; their workspace
  // (per-block state shares and per-head totals, all written before they are
  // read, so nothing needs clearing) must fit the static scratch.
  const size_t need = la::noncausal_ws_bytes((int)BH, N, D, M, dtype == LINATTN_BF16);
  if (need > (size_t)LINATTN_NOALLOC_SCRATCH_BYTES) return LINATTN_ERR_WORKSPACE;
  const long long nq = BH * N * D * es, nv = BH * N * M * es;
  const Span sq(q, nq), sk(k, nq), sv(v, nv), so(o, nv);
  for (const Span& x : {sq, sk, sv})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  void* ws = la::noalloc_scratch();
  if (!ws) return LINATTN_ERR_HIP;
  return hip_status(
      la::launch_noncausal(q, k, v, o, (int)BH, N, D, M, dtype == LINATTN_BF16, ws, (hipStream_t)stream));
}

int linattn_decode_step(const void* q, const void* k, const void* v, void* o, float* S, float* z, int B, int H,
                        int D, int M, int dtype, void* stream) {
  int st = check_shape(B, H, 1, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH == 0) return LINATTN_OK;
  if (!q || !k || !v || !o || !S || !z) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, S, z}))) return st;
  const Span sq(q, BH * D * es), sk(k, BH * D * es), sv(v, BH * M * es), so(o, BH * M * es);
  const Span sS(S, BH * D * M * 4), sz(z, BH * D * 4);
  for (const Span& x : {sq, sk, sv, sS, sz})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sz})
    if (sS.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv})
    if (sz.overlaps(x)) return LINATTN_ERR_ALIAS;
  return hip_status(la::launch_decode(q, k, v, o, S, z, (int)BH, D, M, dtype == LINATTN_BF16, (hipStream_t)stream));
}

int softmax_decode_step(const void* q, const void* k, const void* v, void* o, void* Kc, void* Vc, int B, int H,
                        int L, int Lmax, int D, int M, int dtype, void* stream) {
  int st = check_shape(B, H, Lmax, D, M, dtype);
  if (st) return st;
  if (L < 0 || L >= Lmax) return LINATTN_ERR_SHAPE;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH == 0) return LINATTN_OK;
  if (!q || !k || !v || !o || !Kc || !Vc) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, Kc, Vc}))) return st;
  const Span sq(q, BH * D * es), sk(k, BH * D * es), sv(v, BH * M * es), so(o, BH * M * es);
  const Span sK(Kc, BH * Lmax * D * es), sV(Vc, BH * Lmax * M * es);
  for (const Span& x : {sq, sk, sv, sK, sV})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sV})
    if (sK.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv})
    if (sV.overlaps(x)) return LINATTN_ERR_ALIAS;
  return hip_status(la::launch_softmax_decode(q, k, v, o, Kc, Vc, (int)BH, L, Lmax, D, M, dtype == LINATTN_BF16,
                                              (hipStream_t)stream));
}

int linattn_fmap_dim(int fmap, int nu, int D) {
  if (D != 32 && D != 64) return 0;
  if (fmap == LINATTN_FMAP_DPFP && nu >= 1 && nu <= 3) return la::featmap_dim(nu, D);
  if (fmap == LINATTN_FMAP_POLY2 && nu == 0) return la::featmap_dim(4, D);
  return 0;
}

}  // extern "C"

namespace {
// Internal map code of the kernels: DPFP-nu is nu (1..3), the polynomial map 4; 0 if unsupported.
int fmap_code(int fmap, int nu) {
  if (fmap == LINATTN_FMAP_DPFP && nu >= 1 && nu <= 3) return nu;
  if (fmap == LINATTN_FMAP_POLY2 && nu == 0) return 4;
  return 0;
}
}  // namespace

extern "C" {

size_t linattn_fmap_workspace_bytes(int B, int H, int N, int D, int M, int dtype, int fmap, int nu) {
  if (check_shape(B, H, N, D, M, dtype) != LINATTN_OK) return 0;
  const int code = fmap_code(fmap, nu);
  if (!code) return 0;
  return la::featmap_ws_bytes(code, B * H, N, D, M);
}

int linattn_fmap_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D, int M,
                     int dtype, int fmap, int nu, int causal, const float* S0, const float* z0, float* S_out,
                     float* z_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(B, H, N, D, M, dtype);
  if (st) return st;
  const int code = fmap_code(fmap, nu);
  if (!code) return LINATTN_ERR_UNSUPPORTED;
  if (!causal && (S0 || z0)) return LINATTN_ERR_UNSUPPORTED;
  const long long BH = (long long)B * H, es = esize(dtype), C = la::featmap_dim(code, D);
  const long long nq = BH * N * D * es, nv = BH * N * M * es;
  if ((S0 == nullptr) != (z0 == nullptr)) return LINATTN_ERR_NULL;
  if ((S_out == nullptr) != (z_out == nullptr)) return LINATTN_ERR_NULL;
  if (BH * N > 0 && (!q || !k || !v)) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, S0, z0, S_out, z_out, ws}))) return st;
  if (BH * ((N + 63) / 64) * (C / 64) > (long long)INT32_MAX) return LINATTN_ERR_SHAPE;  // grid sizes
  const size_t need = la::featmap_ws_bytes(code, (int)BH, N, D, M);
  if (need > 0 && (!ws || ws_bytes < need)) return LINATTN_ERR_WORKSPACE;
  const Span sq(q, nq), sk(k, nq), sv(v, nv), so(o, o ? nv : 0);
  const Span sS0(S0, BH * C * M * 4), sz0(z0, BH * C * 4), sSo(S_out, BH * C * M * 4), szo(z_out, BH * C * 4);
  const Span sws(ws, (long long)need);
  for (const Span& x : {sq, sk, sv, sS0, sz0, sSo, szo, sws})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& out : {sSo, szo})
    for (const Span& x : {sq, sk, sv, sws})
      if (out.overlaps(x)) return LINATTN_ERR_ALIAS;
  if (sSo.overlaps(szo)) return LINATTN_ERR_ALIAS;
  if ((sSo.overlaps(sS0) && !sSo.same(sS0)) || (szo.overlaps(sz0) && !szo.same(sz0))) return LINATTN_ERR_ALIAS;
  if (sSo.overlaps(sz0) || szo.overlaps(sS0)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sS0, sz0})
    if (sws.overlaps(x)) return LINATTN_ERR_ALIAS;
  if (BH == 0) return LINATTN_OK;
  if (N == 0 && !S_out) return LINATTN_OK;
  return hip_status(la::launch_featmap(code, q, k, v, o, (int)BH, N, D, M, dtype == LINATTN_BF16, causal ? 1 : 0,
                                       S0, z0, S_out, z_out, ws, (hipStream_t)stream));
}

size_t deltanet_workspace_bytes(int B, int H, int N, int D, int M, int dtype) {
  if (check_shape(B, H, N, D, M, dtype) != LINATTN_OK) return 0;
  return la::deltanet_ws_bytes(B * H, N, D, M);
}

int deltanet_fwd(const void* q, const void* k, const void* v, const void* beta, void* o, int B, int H, int N, int D,
                 int M, int dtype, const float* W0, float* W_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(B, H, N, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH * N > 0 && (!q || !k || !v || !beta || !o)) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, W0, W_out, ws}))) return st;
  if ((st = check_align_elem(beta, (int)es))) return st;
  const size_t need = la::deltanet_ws_bytes((int)BH, N, D, M);
  if (need > 0 && (!ws || ws_bytes < need)) return LINATTN_ERR_WORKSPACE;
  const long long nq = BH * N * D * es, nv = BH * N * M * es;
  const Span sq(q, nq), sk(k, nq), sv(v, nv), sb(beta, BH * N * es), so(o, nv);
  const Span sW0(W0, BH * M * D * 4), sWo(W_out, BH * M * D * 4), sws(ws, (long long)need);
  for (const Span& x : {sq, sk, sv, sb, sW0, sWo, sws})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sb, sws})
    if (sWo.overlaps(x)) return LINATTN_ERR_ALIAS;
  if (sWo.overlaps(sW0) && !sWo.same(sW0)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sb, sW0})
    if (sws.overlaps(x)) return LINATTN_ERR_ALIAS;
  if (BH == 0 || (N == 0 && !W_out)) return LINATTN_OK;
  return hip_status(la::launch_deltanet(q, k, v, beta, o, (int)BH, N, D, M, dtype == LINATTN_BF16, W0, W_out,
                                        need > 0 ? ws : nullptr, (hipStream_t)stream));
}

int deltanet_decode_step(const void* q, const void* k, const void* v, const void* beta, void* o, float* W, int B,
                         int H, int D, int M, int dtype, void* stream) {
  int st = check_shape(B, H, 1, D, M, dtype);
  if (st) return st;
  const long long BH = (long long)B * H, es = esize(dtype);
  if (BH == 0) return LINATTN_OK;
  if (!q || !k || !v || !beta || !o || !W) return LINATTN_ERR_NULL;
  if ((st = check_align({q, k, v, o, W}))) return st;
  if ((st = check_align_elem(beta, (int)es))) return st;
  const Span sq(q, BH * D * es), sk(k, BH * D * es), sv(v, BH * M * es), sb(beta, BH * es), so(o, BH * M * es);
  const Span sW(W, BH * M * D * 4);
  for (const Span& x : {sq, sk, sv, sb, sW})
    if (so.overlaps(x)) return LINATTN_ERR_ALIAS;
  for (const Span& x : {sq, sk, sv, sb})
    if (sW.overlaps(x)) return LINATTN_ERR_ALIAS;
  return hip_status(
      la::launch_deltanet_step(q, k, v, beta, o, W, (int)BH, D, M, dtype == LINATTN_BF16, (hipStream_t)stream));
}

const char* linattn_status_str(int status) {
  switch (status) {
    case LINATTN_OK: return "LINATTN_OK";
    case LINATTN_ERR_NULL: return "LINATTN_ERR_NULL";
    case LINATTN_ERR_SHAPE: return "LINATTN_ERR_SHAPE";
    case LINATTN_ERR_DTYPE: return "LINATTN_ERR_DTYPE";
    case LINATTN_ERR_UNSUPPORTED: return "LINATTN_ERR_UNSUPPORTED";
    case LINATTN_ERR_ALIGN: return "LINATTN_ERR_ALIGN";
    case LINATTN_ERR_ALIAS: return "LINATTN_ERR_ALIAS";
    case LINATTN_ERR_WORKSPACE: return "LINATTN_ERR_WORKSPACE";
    case LINATTN_ERR_HIP: return "LINATTN_ERR_HIP";
    default: return "LINATTN_ERR_UNKNOWN";
  }
}

int linattn_abi_version(void) { return LINATTN_ABI_VERSION; }

}  // extern "C"
