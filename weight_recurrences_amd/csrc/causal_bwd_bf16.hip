// Backward of causal linear attention for bf16 inputs on gfx950 (bf16 MFMA).
//
// "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器", §3.3 eq.(9)-(12) and §3.3.1 (gradients as cumulative sums).  The
// gradient formulas are those of the float32 path (causal_bwd.hip): with
// num_i = S_i^T phi(q_i), den_i = z_i . phi(q_i),
//   a_i = dO_i / den_i,   b_i = -(dO_i . num_i) / den_i^2,
//   dphi(q_i) = S_i a_i + z_i b_i + sum_{j in chunk, j<=i} E[i][j] phi(k_j),
//   dphi(k_j) = R_j v_j + r_j + sum_{i in chunk, i>=j} E[i][j] phi(q_i),
//   dv_j      = R_j^T phi(k_j) + sum_{i in chunk, i>=j} P[i][j] a_i,
// E[i][j] = a_i . v_j + b_i, P[i][j] = phi(q_i) . phi(k_j), (S, z) the prefix
// state before the chunk and (R, r) = sums over the later tokens of
// phi(q_i) a_i^T and phi(q_i) b_i.
//
// Every product is a 16x16x32 bf16 MFMA tile, and every operand that is not
// an exact bf16 input enters as a bf16 head and tail (x = hi + lo to about
// 2^-17; the tail x tail product is dropped), with float32 accumulation.  The
// gradients are differences of nearly equal terms: b_i = -a_i . o_i cancels
// against S a_i in dphi(q) and against a_i . v_j in E, and E sums to zero
// against P[i][j] over j, so sum_j E[i][j] phi(k_j) cancels too (for a single
// token dq is exactly 0).  One bf16 rounding of a, P, E or phi in those
// products leaves errors of order 2^-9 of the cancelled terms, several times
// the bf16 rounding of the result; an emulation of the roundings pinned
// which operands need the tail.
//
// Tile layouts (lane l = 16 g + n; MFMA A: row n, k = 8g..8g+7 of a 32-slab;
// B: column n, same k; result: rows 4g + r of column n):
//  * contraction over d or m in natural order: 16-byte unit reads of
//    row-major tiles (unit16);
//  * contraction over tokens or m in the permuted order k = 32s + 16h + 4g + r:
//    an accumulator tile pair (h = 0, 1) is directly the B operand, and the
//    matching A operand comes from ds_read_b64_tr_b16 (jfrag) or two 8-byte
//    reads (unit8).
// Transposed state tiles St[m][d] (head and tail) serve both as the A operand
// of S^T phi(q) (unit reads) and of S a (transposed reads).
//
// Kernels (the block prefix states come from the forward block kernels):
//   bwd_q_bf16_kernel       forward sweep per block: 1/den and b per token, dq
//   bwd_rstate_bf16_kernel  per block: sum phi(q_i) a_i^T and sum phi(q_i) b_i
//   bwd_kv_bf16_kernel      reverse sweep per block: dk, dv
// a_i is never stored: the later kernels rebuild it from dO and 1/den.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace la {
namespace bwdh {

constexpr int NT = 256;
constexpr int C = 64;

template <int D, int M>
struct G {
  static constexpr int TD = D / 16, TM = M / 16;
  static constexpr int WPT = 4 / TD;    // waves sharing a d-tile of a state
  static constexpr int TMW = TM / WPT;  // m-tiles of a state per wave
  static constexpr int UD = D / 8, UM = M / 8;  // 16-byte units per row
  static constexpr int SD = D / 32, SM = M / 32;  // 32-wide slabs
  static constexpr int KU = C * UD / NT, VU = C * UM / NT;  // units per thread per tile
};

template <int D, int M>
__device__ __forceinline__ void tile_coords(int w, int u, int& td, int& tm) {
  td = w % G<D, M>::TD;
  tm = w / G<D, M>::TD + G<D, M>::WPT * u;
}

// Rows [0, nt) of a [*, W] bf16 tensor into registers, one 16-byte unit per
// slot; rows past nt read as zeros.
template <int W, int NU>
__device__ __forceinline__ void fetch(u32x4 (&r)[NU], const bf16_t* src, int nt, int tid) {
  constexpr int U = W / 8;
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int p = tid + NT * i, row = p / U, cu = p % U;
    r[i] = row < nt ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)row * W + cu * 8))
                    : u32x4{0u, 0u, 0u, 0u};
  }
}

// Raw units into a swizzled tile.
template <int W, int NU>
__device__ __forceinline__ void put_raw(bf16_t* tile, const u32x4 (&r)[NU], int tid) {
  constexpr int U = W / 8;
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int p = tid + NT * i;
    unit16<U>(tile, p / U, (p % U) * 8) = r[i];
  }
}

// phi of the units: head into `hi`, tail into `lo` (when given); rows at or
// past nt give zeros.
template <int W, int NU, bool TAIL>
__device__ __forceinline__ void put_phi(bf16_t* hi, bf16_t* lo, const u32x4 (&r)[NU], int nt, int tid) {
  constexpr int U = W / 8;
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int p = tid + NT * i, row = p / U, cu = p % U;
    u32x4 hv, lv;
    phi_split8(r[i], row < nt, hv, lv);
    unit16<U>(hi, row, cu * 8) = hv;
    if (TAIL) unit16<U>(lo, row, cu * 8) = lv;
  }
}

// 1/den of the row of each unit slot (zero past the end).
template <int W, int NU>
__device__ __forceinline__ void fetch_scale(float (&sc)[NU], const float* inv, int nt, int tid) {
  constexpr int U = W / 8;
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int row = (tid + NT * i) / U;
    sc[i] = row < nt ? inv[row] : 0.f;
  }
}

// a = dO * (1/den) of the units, split into head and tail.
template <int W, int NU>
__device__ __forceinline__ void put_scaled(bf16_t* hi, bf16_t* lo, const u32x4 (&r)[NU], const float (&sc)[NU],
                                           int tid) {
  constexpr int U = W / 8;
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int p = tid + NT * i, row = p / U, cu = p % U;
    const float s = sc[i];
    u32x4 hv, lv;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float a = lo_of(r[i][h]) * s, b = hi_of(r[i][h]) * s;
      const uint32_t hp = cvt_pk(a, b);
      hv[h] = hp;
      lv[h] = cvt_pk(a - lo_of(hp), b - hi_of(hp));
    }
    unit16<U>(hi, row, cu * 8) = hv;
    unit16<U>(lo, row, cu * 8) = lv;
  }
}

// A state tile set (float32 accumulators): wave w holds tiles (td, tm) of
// tile_coords, element r of tile u is X[16 td + 4g + r][16 tm + n]; x holds the
// vector part x[16 td + 4g + r] (kept by waves w < D/16, computed by all).
template <int D, int M>
struct State {
  f32x4 S[G<D, M>::TMW];
  f32x4 x;
};

template <int D, int M>
__device__ __forceinline__ void state_load(State<D, M>& st, const float* S, const float* x, int w, int n, int g) {
#pragma unroll
  for (int u = 0; u < G<D, M>::TMW; ++u) {
    int td, tm;
    tile_coords<D, M>(w, u, td, tm);
#pragma unroll
    for (int r = 0; r < 4; ++r) st.S[u][r] = S[(16 * td + 4 * g + r) * M + 16 * tm + n];
  }
  const int td = w % G<D, M>::TD;
#pragma unroll
  for (int r = 0; r < 4; ++r) st.x[r] = x[16 * td + 4 * g + r];
}

// Transposed head/tail copies St[m][d] of the state and its vector part in
// float32.
template <int D, int M>
__device__ __forceinline__ void state_stage(const State<D, M>& st, bf16_t* Th, bf16_t* Tl, float* xs, int w, int n,
                                            int g) {
  using GG = G<D, M>;
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) {
    int td, tm;
    tile_coords<D, M>(w, u, td, tm);
    const f32x4 x = st.S[u];
    const uint32_t h0 = cvt_pk(x[0], x[1]), h1 = cvt_pk(x[2], x[3]);
    unit8<GG::UD>(Th, 16 * tm + n, 16 * td + 4 * g) = u32x2{h0, h1};
    unit8<GG::UD>(Tl, 16 * tm + n, 16 * td + 4 * g) =
        u32x2{cvt_pk(x[0] - lo_of(h0), x[1] - hi_of(h0)), cvt_pk(x[2] - lo_of(h1), x[3] - hi_of(h1))};
  }
  if (w < GG::TD && n == 0) *reinterpret_cast<f32x4*>(&xs[16 * w + 4 * g]) = st.x;
}

// Two accumulator tiles (h = 0, 1) as one bf16 B operand over the permuted
// k = 16 h + 4 g + r.
__device__ __forceinline__ bf16x8 pair_frag(const f32x4& t0, const f32x4& t1) {
  return as_bf16x8(u32x4{cvt_pk(t0[0], t0[1]), cvt_pk(t0[2], t0[3]), cvt_pk(t1[0], t1[1]), cvt_pk(t1[2], t1[3])});
}

// The same pair split into head and tail.
__device__ __forceinline__ void pair_frag_split(const f32x4& t0, const f32x4& t1, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
  h[0] = cvt_pk(t0[0], t0[1]);
  h[1] = cvt_pk(t0[2], t0[3]);
  h[2] = cvt_pk(t1[0], t1[1]);
  h[3] = cvt_pk(t1[2], t1[3]);
  l[0] = cvt_pk(t0[0] - lo_of(h[0]), t0[1] - hi_of(h[0]));
  l[1] = cvt_pk(t0[2] - lo_of(h[1]), t0[3] - hi_of(h[1]));
  l[2] = cvt_pk(t1[0] - lo_of(h[2]), t1[1] - hi_of(h[2]));
  l[3] = cvt_pk(t1[2] - lo_of(h[3]), t1[3] - hi_of(h[3]));
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// Row `row` of a swizzled tile at the permuted columns 32s + 16h + 4g + r.
template <int U>
__device__ __forceinline__ bf16x8 perm_row(bf16_t* tile, int row, int s, int g) {
  const u32x2 a = unit8<U>(tile, row, 32 * s + 4 * g), b = unit8<U>(tile, row, 32 * s + 16 + 4 * g);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// A broadcast vector (every row of A equal to x) at k = 32s + 8g + e, split
// into head and tail.
__device__ __forceinline__ void vec_frag(const float* x, int s, int g, bf16x8& hi, bf16x8& lo) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(&x[32 * s + 8 * g]);
  const f32x4 b = *reinterpret_cast<const f32x4*>(&x[32 * s + 8 * g + 4]);
  u32x4 h, l;
  h[0] = cvt_pk(a[0], a[1]);
  h[1] = cvt_pk(a[2], a[3]);
  h[2] = cvt_pk(b[0], b[1]);
  h[3] = cvt_pk(b[2], b[3]);
  l[0] = cvt_pk(a[0] - lo_of(h[0]), a[1] - hi_of(h[0]));
  l[1] = cvt_pk(a[2] - lo_of(h[1]), a[3] - hi_of(h[1]));
  l[2] = cvt_pk(b[0] - lo_of(h[2]), b[1] - hi_of(h[2]));
  l[3] = cvt_pk(b[2] - lo_of(h[3]), b[3] - hi_of(h[3]));
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// A B operand whose column is the same for every n: x at the permuted
// k = 32s + 16h + 4g + r, head and tail.
__device__ __forceinline__ void perm_vec_frag(const float* x, int s, int g, bf16x8& hi, bf16x8& lo) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(&x[32 * s + 4 * g]);
  const f32x4 b = *reinterpret_cast<const f32x4*>(&x[32 * s + 16 + 4 * g]);
  u32x4 h, l;
  h[0] = cvt_pk(a[0], a[1]);
  h[1] = cvt_pk(a[2], a[3]);
  h[2] = cvt_pk(b[0], b[1]);
  h[3] = cvt_pk(b[2], b[3]);
  l[0] = cvt_pk(a[0] - lo_of(h[0]), a[1] - hi_of(h[0]));
  l[1] = cvt_pk(a[2] - lo_of(h[1]), a[3] - hi_of(h[1]));
  l[2] = cvt_pk(b[0] - lo_of(h[2]), b[1] - hi_of(h[2]));
  l[3] = cvt_pk(b[2] - lo_of(h[3]), b[3] - hi_of(h[3]));
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ float4 raw4(const u32x2& w) {
  return float4{lo_of(w[0]), hi_of(w[0]), lo_of(w[1]), hi_of(w[1])};
}
__device__ __forceinline__ float dphi_raw(float x) { return x > 0.f ? 1.f : __expf(x); }

// ----------------------------------------------------------------------------
// Forward sweep.  Grid BH * nblk; wave w owns the query rows i = 16 w + n of
// each chunk.  Every MFMA runs unconditionally (masks are selects), so no
// branch separates an MFMA from a read of its result.
template <int D, int M>
struct SmemQ {
  bf16_t Kh[C * D], Kl[C * D];  // phi(K) head / tail
  bf16_t Vs[C * M];
  bf16_t Qs[C * D];             // raw q
  bf16_t Gs[C * M];             // raw dO
  bf16_t Sh[M * D], Sl[M * D];  // S^T head / tail
  float Zs[D];
};

template <int D, int M>
__global__ __launch_bounds__(NT, 2) void bwd_q_bf16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                           const bf16_t* __restrict__ v, const bf16_t* __restrict__ dO,
                                                           bf16_t* __restrict__ dq, int N, int tblk, int nblk,
                                                           const float* __restrict__ preS,
                                                           const float* __restrict__ preZ, float* __restrict__ inv_ws,
                                                           float* __restrict__ b_ws) {
  using GG = G<D, M>;
  __shared__ __attribute__((aligned(16))) SmemQ<D, M> sm;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const int td = w % GG::TD;
  const bf16x8 ones = ones8();
  const int i_loc = 16 * w + n;

  State<D, M> st;
  {
    const size_t rec = (size_t)bh * nblk + blk;
    state_load<D, M>(st, preS + rec * D * M, preZ + rec * D, w, n, g);
  }
  u32x4 rk[GG::KU], rv[GG::VU], rq[GG::KU], rg[GG::VU];
  {
    const size_t row0 = (size_t)bh * N + t0;
    const int nt = min(C, t1 - t0);
    fetch<D>(rk, k + row0 * D, nt, tid);
    fetch<M>(rv, v + row0 * M, nt, tid);
    fetch<D>(rq, q + row0 * D, nt, tid);
    fetch<M>(rg, dO + row0 * M, nt, tid);
  }

  for (int c0 = t0; c0 < t1; c0 += C) {
    const int nt = min(C, t1 - c0);
    const size_t row0 = (size_t)bh * N + c0;
    __syncthreads();  // the previous chunk's readers are done
    put_phi<D, GG::KU, true>(sm.Kh, sm.Kl, rk, nt, tid);
    put_raw<M>(sm.Vs, rv, tid);
    put_raw<D>(sm.Qs, rq, tid);
    put_raw<M>(sm.Gs, rg, tid);
    state_stage<D, M>(st, sm.Sh, sm.Sl, sm.Zs, w, n, g);
    __syncthreads();
    if (c0 + C < t1) {  // next chunk's loads, in flight during this chunk
      const int nn = min(C, t1 - c0 - C);
      fetch<D>(rk, k + (row0 + C) * D, nn, tid);
      fetch<M>(rv, v + (row0 + C) * M, nn, tid);
      fetch<D>(rq, q + (row0 + C) * D, nn, tid);
      fetch<M>(rg, dO + (row0 + C) * M, nn, tid);
    }

    // The forward quantities num, den (and so o_i and b_i) are formed to
    // float32 level: phi(q_i), phi(K), the state and P all enter as head and
    // tail, because b_i cancels against S a_i in dphi(q) and against a_i . v_j
    // in E.
    // phi(q_i) as B operand, d = 32s + 8g + e, head and tail.
    bf16x8 qf[GG::SD], qfl[GG::SD];
#pragma unroll
    for (int s = 0; s < GG::SD; ++s) {
      u32x4 hv, lv;
      phi_split8(unit16<GG::UD>((const bf16_t*)sm.Qs, i_loc, 32 * s + 8 * g), true, hv, lv);
      qf[s] = as_bf16x8(hv);
      qfl[s] = as_bf16x8(lv);
    }
    // (1) PT[jt][r] = P[i][j], j = 16 jt + 4g + r, zero where j > i.
    f32x4 PT[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SD; ++s) {
        const bf16x8 kh = as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Kh, 16 * jt + n, 32 * s + 8 * g));
        acc = mma(kh, qf[s], acc);
        acc = mma(kh, qfl[s], acc);
        acc = mma(as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Kl, 16 * jt + n, 32 * s + 8 * g)), qf[s], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) PT[jt][r] = (16 * jt + 4 * g + r <= i_loc) ? acc[r] : 0.f;
    }
    bf16x8 pf0, pf0l, pf1, pf1l;
    pair_frag_split(PT[0], PT[1], pf0, pf0l);
    pair_frag_split(PT[2], PT[3], pf1, pf1l);
    // (2) numT[mt][r] = num[i][m], m = 16 mt + 4g + r: S^T phi(q_i) + V^T P^T.
    f32x4 numT[GG::TM];
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SD; ++s) {
        const bf16x8 sh = as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Sh, 16 * mt + n, 32 * s + 8 * g));
        acc = mma(sh, qf[s], acc);
        acc = mma(sh, qfl[s], acc);
        acc = mma(as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Sl, 16 * mt + n, 32 * s + 8 * g)), qf[s], acc);
      }
      const bf16x8 v0 = jfrag<GG::UM>(sm.Vs, 0, 16 * mt, g, n), v1 = jfrag<GG::UM>(sm.Vs, 32, 16 * mt, g, n);
      acc = mma(v0, pf0, acc);
      acc = mma(v0, pf0l, acc);
      acc = mma(v1, pf1, acc);
      acc = mma(v1, pf1l, acc);
      numT[mt] = acc;
    }
    // (3) den_i = z . phi(q_i) + sum_j P[i][j] (every row of the tile).
    float den;
    {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SD; ++s) {
        bf16x8 zh, zl;
        vec_frag(sm.Zs, s, g, zh, zl);
        acc = mma(zh, qf[s], acc);
        acc = mma(zh, qfl[s], acc);
        acc = mma(zl, qf[s], acc);
      }
      acc = mma(ones, pf0, acc);
      acc = mma(ones, pf0l, acc);
      acc = mma(ones, pf1, acc);
      acc = mma(ones, pf1l, acc);
      den = acc[0];
    }
    // (4) a_i = dO_i / den_i, b_i = -(dO_i . num_i) / den_i^2.
    const bool rowok = i_loc < nt;
    const float inv = rowok ? 1.f / den : 0.f;
    f32x4 aT[GG::TM];
    float bp = 0.f;
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt) {
      const float4 go = raw4(unit8<GG::UM>(sm.Gs, i_loc, 16 * mt + 4 * g));
      aT[mt] = f32x4{go.x * inv, go.y * inv, go.z * inv, go.w * inv};
      bp += go.x * numT[mt][0] + go.y * numT[mt][1] + go.z * numT[mt][2] + go.w * numT[mt][3];
    }
    bp += __shfl_xor(bp, 16);
    bp += __shfl_xor(bp, 32);
    const float b = -bp * inv * inv;
    if (rowok && g == 0) {
      inv_ws[row0 + i_loc] = inv;
      b_ws[row0 + i_loc] = b;
    }
    bf16x8 af[GG::SM], afl[GG::SM];  // a_i head / tail, m = 32s + 16h + 4g + r
#pragma unroll
    for (int s = 0; s < GG::SM; ++s) pair_frag_split(aT[2 * s], aT[2 * s + 1], af[s], afl[s]);
    // (5) ET[jt][r] = E[i][j] = a_i . v_j + b_i, zero where j > i.
    f32x4 ET[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SM; ++s) {
        const bf16x8 vrow = perm_row<GG::UM>(sm.Vs, 16 * jt + n, s, g);
        acc = mma(vrow, af[s], acc);
        acc = mma(vrow, afl[s], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ET[jt][r] = (16 * jt + 4 * g + r <= i_loc) ? acc[r] + b : 0.f;
    }
    bf16x8 ef0, ef0l, ef1, ef1l;
    pair_frag_split(ET[0], ET[1], ef0, ef0l);
    pair_frag_split(ET[2], ET[3], ef1, ef1l);
    // (6) dphi(q_i)[d] = (S a_i)[d] + z_d b_i + sum_j E[i][j] phi(k_j)[d];  dq = dphi(q) phi'(q).
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SM; ++s) {
        const bf16x8 sh = jfrag<GG::UD>(sm.Sh, 32 * s, 16 * dt, g, n);
        acc = mma(sh, af[s], acc);
        acc = mma(sh, afl[s], acc);
        acc = mma(jfrag<GG::UD>(sm.Sl, 32 * s, 16 * dt, g, n), af[s], acc);
      }
      {  // sum_j E[i][j] phi(k_j): E sums to zero against P[i][j], so both as head and tail
        const bf16x8 k0 = jfrag<GG::UD>(sm.Kh, 0, 16 * dt, g, n), k1 = jfrag<GG::UD>(sm.Kh, 32, 16 * dt, g, n);
        acc = mma(k0, ef0, acc);
        acc = mma(k0, ef0l, acc);
        acc = mma(jfrag<GG::UD>(sm.Kl, 0, 16 * dt, g, n), ef0, acc);
        acc = mma(k1, ef1, acc);
        acc = mma(k1, ef1l, acc);
        acc = mma(jfrag<GG::UD>(sm.Kl, 32, 16 * dt, g, n), ef1, acc);
      }
      const f32x4 zz = *reinterpret_cast<const f32x4*>(&sm.Zs[16 * dt + 4 * g]);
      const float4 qq = raw4(unit8<GG::UD>(sm.Qs, i_loc, 16 * dt + 4 * g));
      const float o0 = (acc[0] + zz[0] * b) * dphi_raw(qq.x), o1 = (acc[1] + zz[1] * b) * dphi_raw(qq.y);
      const float o2 = (acc[2] + zz[2] * b) * dphi_raw(qq.z), o3 = (acc[3] + zz[3] * b) * dphi_raw(qq.w);
      if (rowok)
        *reinterpret_cast<u32x2*>(dq + (row0 + i_loc) * D + 16 * dt + 4 * g) = u32x2{cvt_pk(o0, o1), cvt_pk(o2, o3)};
    }
    // (7) S += phi(K)^T V, z += colsum phi(K) (head and tail of phi(K)).
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 ah = jfrag<GG::UD>(sm.Kh, 32 * s, 16 * td, g, n);
      const bf16x8 al = jfrag<GG::UD>(sm.Kl, 32 * s, 16 * td, g, n);
#pragma unroll
      for (int u = 0; u < GG::TMW; ++u) {
        int tdd, tm;
        tile_coords<D, M>(w, u, tdd, tm);
        const bf16x8 bv = jfrag<GG::UM>(sm.Vs, 32 * s, 16 * tm, g, n);
        st.S[u] = mma(ah, bv, st.S[u]);
        st.S[u] = mma(al, bv, st.S[u]);
      }
      st.x = mma(ah, ones, st.x);
      st.x = mma(al, ones, st.x);
    }
  }
}

// ----------------------------------------------------------------------------
// Per-block suffix contributions R_b = sum_i phi(q_i) a_i^T, r_b = sum_i
// phi(q_i) b_i into suf[bh][blk] ([D][M] then [D], float32).
template <int D, int M>
struct SmemR {
  bf16_t Qh[C * D], Ql[C * D];
  bf16_t Ah[C * M], Al[C * M];
  float Bs[C];
};

// R += phi(Q)^T a, r += phi(Q)^T b over one chunk in LDS (head x head, head x
// tail and tail x head products).
template <int D, int M>
__device__ __forceinline__ void rstate_update(State<D, M>& st, bf16_t* Qh, bf16_t* Ql, bf16_t* Ah, bf16_t* Al,
                                              const float* Bs, int w, int n, int g) {
  using GG = G<D, M>;
  const int td = w % GG::TD;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const bf16x8 qh = jfrag<GG::UD>(Qh, 32 * s, 16 * td, g, n);
    const bf16x8 ql = jfrag<GG::UD>(Ql, 32 * s, 16 * td, g, n);
#pragma unroll
    for (int u = 0; u < GG::TMW; ++u) {
      int tdd, tm;
      tile_coords<D, M>(w, u, tdd, tm);
      const bf16x8 ah = jfrag<GG::UM>(Ah, 32 * s, 16 * tm, g, n);
      const bf16x8 al = jfrag<GG::UM>(Al, 32 * s, 16 * tm, g, n);
      st.S[u] = mma(qh, ah, st.S[u]);
      st.S[u] = mma(qh, al, st.S[u]);
      st.S[u] = mma(ql, ah, st.S[u]);
    }
    bf16x8 bh, bl;
    perm_vec_frag(Bs, s, g, bh, bl);
    st.x = mma(qh, bh, st.x);
    st.x = mma(qh, bl, st.x);
    st.x = mma(ql, bh, st.x);
  }
}

template <int D, int M>
__global__ __launch_bounds__(NT, 2) void bwd_rstate_bf16_kernel(const bf16_t* __restrict__ q,
                                                                const bf16_t* __restrict__ dO,
                                                                const float* __restrict__ inv_ws,
                                                                const float* __restrict__ b_ws, int N, int tblk,
                                                                int nblk, float* __restrict__ suf) {
  using GG = G<D, M>;
  __shared__ __attribute__((aligned(16))) SmemR<D, M> sm;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  State<D, M> st;
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) st.S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.x = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 rq[GG::KU], rg[GG::VU];
  float sc[GG::VU], rb = 0.f;
  {
    const size_t row0 = (size_t)bh * N + t0;
    const int nt = min(C, t1 - t0);
    fetch<D>(rq, q + row0 * D, nt, tid);
    fetch<M>(rg, dO + row0 * M, nt, tid);
    fetch_scale<M>(sc, inv_ws + row0, nt, tid);
    if (tid < nt) rb = b_ws[row0 + tid];
  }
  for (int c0 = t0; c0 < t1; c0 += C) {
    const int nt = min(C, t1 - c0);
    const size_t row0 = (size_t)bh * N + c0;
    __syncthreads();  // the previous chunk's readers are done
    put_phi<D, GG::KU, true>(sm.Qh, sm.Ql, rq, nt, tid);
    put_scaled<M, GG::VU>(sm.Ah, sm.Al, rg, sc, tid);
    if (tid < C) sm.Bs[tid] = rb;
    __syncthreads();
    if (c0 + C < t1) {  // next chunk's loads, in flight during this chunk
      const int nn = min(C, t1 - c0 - C);
      fetch<D>(rq, q + (row0 + C) * D, nn, tid);
      fetch<M>(rg, dO + (row0 + C) * M, nn, tid);
      fetch_scale<M>(sc, inv_ws + row0 + C, nn, tid);
      rb = tid < nn ? b_ws[row0 + C + tid] : 0.f;
    }
    rstate_update<D, M>(st, sm.Qh, sm.Ql, sm.Ah, sm.Al, sm.Bs, w, n, g);
  }
  float* dst = suf + ((size_t)bh * nblk + blk) * (D * M + D);
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) {
    int td, tm;
    tile_coords<D, M>(w, u, td, tm);
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * td + 4 * g + r) * M + 16 * tm + n] = st.S[u][r];
  }
  if (w < GG::TD && n == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[D * M + 16 * w + 4 * g + r] = st.x[r];
  }
}

// ----------------------------------------------------------------------------
// Reverse sweep.  Grid BH * nblk; the block's suffix state is suf[bh][blk];
// chunks run from the last to the first and wave w owns the key rows
// j = 16 w + n.
template <int D, int M>
struct SmemKV {
  bf16_t Qh[C * D], Ql[C * D];  // phi(Q) head / tail
  bf16_t Kr[C * D];             // raw k
  bf16_t Vs[C * M];
  bf16_t Ah[C * M], Al[C * M];  // a head / tail
  bf16_t Rh[M * D], Rl[M * D];  // R^T head / tail
  float Bs[C];
  float rs[D];
};

template <int D, int M>
__global__ __launch_bounds__(NT, 2) void bwd_kv_bf16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                            const bf16_t* __restrict__ v,
                                                            const bf16_t* __restrict__ dO,
                                                            const float* __restrict__ inv_ws,
                                                            const float* __restrict__ b_ws, bf16_t* __restrict__ dk,
                                                            bf16_t* __restrict__ dv, int N, int tblk, int nblk,
                                                            const float* __restrict__ suf) {
  using GG = G<D, M>;
  __shared__ __attribute__((aligned(16))) SmemKV<D, M> sm;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const int j_loc = 16 * w + n;
  const int nchb = (t1 - t0 + C - 1) / C;

  State<D, M> st;
  {
    const float* src = suf + ((size_t)bh * nblk + blk) * (D * M + D);
    state_load<D, M>(st, src, src + D * M, w, n, g);
  }
  u32x4 rq[GG::KU], rk[GG::KU], rv[GG::VU], rg[GG::VU];
  float sc[GG::VU], rb = 0.f;
  {
    const int c0 = t0 + (nchb - 1) * C;
    const size_t row0 = (size_t)bh * N + c0;
    const int nt = min(C, t1 - c0);
    fetch<D>(rq, q + row0 * D, nt, tid);
    fetch<D>(rk, k + row0 * D, nt, tid);
    fetch<M>(rv, v + row0 * M, nt, tid);
    fetch<M>(rg, dO + row0 * M, nt, tid);
    fetch_scale<M>(sc, inv_ws + row0, nt, tid);
    if (tid < nt) rb = b_ws[row0 + tid];
  }

  for (int ci = nchb - 1; ci >= 0; --ci) {
    const int c0 = t0 + ci * C;
    const int nt = min(C, t1 - c0);
    const size_t row0 = (size_t)bh * N + c0;
    __syncthreads();  // the previous chunk's readers are done
    put_phi<D, GG::KU, true>(sm.Qh, sm.Ql, rq, nt, tid);
    put_raw<D>(sm.Kr, rk, tid);
    put_raw<M>(sm.Vs, rv, tid);
    put_scaled<M, GG::VU>(sm.Ah, sm.Al, rg, sc, tid);
    if (tid < C) sm.Bs[tid] = rb;
    state_stage<D, M>(st, sm.Rh, sm.Rl, sm.rs, w, n, g);
    __syncthreads();
    if (ci > 0) {  // the preceding chunk's loads (always full), in flight during this chunk
      const size_t prow = row0 - C;
      fetch<D>(rq, q + prow * D, C, tid);
      fetch<D>(rk, k + prow * D, C, tid);
      fetch<M>(rv, v + prow * M, C, tid);
      fetch<M>(rg, dO + prow * M, C, tid);
      fetch_scale<M>(sc, inv_ws + prow, C, tid);
      rb = tid < C ? b_ws[prow + tid] : 0.f;
    }

    // Key row j operand: phi(k_j) head and tail (d natural).
    const bool rowok = j_loc < nt;
    bf16x8 kf[GG::SD], kfl[GG::SD];
#pragma unroll
    for (int s = 0; s < GG::SD; ++s) {
      u32x4 hv, lv;
      phi_split8(unit16<GG::UD>((const bf16_t*)sm.Kr, j_loc, 32 * s + 8 * g), rowok, hv, lv);
      kf[s] = as_bf16x8(hv);
      kfl[s] = as_bf16x8(lv);
    }
    // (1) PJ[it][r] = P[i][j], i = 16 it + 4g + r, zero where i < j.  P and then
    // E are formed just before their products, which keeps the live registers
    // below the two-workgroups-per-CU budget.
    bf16x8 pj0, pj0l, pj1, pj1l;
    {
      f32x4 PJ[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 p{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < GG::SD; ++s) {
          const bf16x8 qh = as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Qh, 16 * it + n, 32 * s + 8 * g));
          p = mma(qh, kf[s], p);
          p = mma(qh, kfl[s], p);
          p = mma(as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Ql, 16 * it + n, 32 * s + 8 * g)), kf[s], p);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) PJ[it][r] = (16 * it + 4 * g + r >= j_loc) ? p[r] : 0.f;
      }
      pair_frag_split(PJ[0], PJ[1], pj0, pj0l);
      pair_frag_split(PJ[2], PJ[3], pj1, pj1l);
    }
    // (3) dv_j[m] = (R^T phi(k_j))[m] + sum_i P[i][j] a_i[m].
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SD; ++s) {
        const bf16x8 rh = as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Rh, 16 * mt + n, 32 * s + 8 * g));
        acc = mma(rh, kf[s], acc);
        acc = mma(rh, kfl[s], acc);
        acc = mma(as_bf16x8(unit16<GG::UD>((const bf16_t*)sm.Rl, 16 * mt + n, 32 * s + 8 * g)), kf[s], acc);
      }
      {
        const bf16x8 a0 = jfrag<GG::UM>(sm.Ah, 0, 16 * mt, g, n), a1 = jfrag<GG::UM>(sm.Ah, 32, 16 * mt, g, n);
        acc = mma(a0, pj0, acc);
        acc = mma(a0, pj0l, acc);
        acc = mma(jfrag<GG::UM>(sm.Al, 0, 16 * mt, g, n), pj0, acc);
        acc = mma(a1, pj1, acc);
        acc = mma(a1, pj1l, acc);
        acc = mma(jfrag<GG::UM>(sm.Al, 32, 16 * mt, g, n), pj1, acc);
      }
      if (rowok)
        *reinterpret_cast<u32x2*>(dv + (row0 + j_loc) * M + 16 * mt + 4 * g) =
            u32x2{cvt_pk(acc[0], acc[1]), cvt_pk(acc[2], acc[3])};
    }
    // (2) EJ[it][r] = E[i][j] = a_i . v_j + b_i, zero where i < j.
    bf16x8 ej0, ej0l, ej1, ej1l;
    {
      f32x4 EJ[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 e{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < GG::SM; ++s) {
          const bf16x8 vf = as_bf16x8(unit16<GG::UM>((const bf16_t*)sm.Vs, j_loc, 32 * s + 8 * g));  // v_j
          e = mma(as_bf16x8(unit16<GG::UM>((const bf16_t*)sm.Ah, 16 * it + n, 32 * s + 8 * g)), vf, e);
          e = mma(as_bf16x8(unit16<GG::UM>((const bf16_t*)sm.Al, 16 * it + n, 32 * s + 8 * g)), vf, e);
        }
        const f32x4 bb = *reinterpret_cast<const f32x4*>(&sm.Bs[16 * it + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) EJ[it][r] = (16 * it + 4 * g + r >= j_loc) ? e[r] + bb[r] : 0.f;
      }
      pair_frag_split(EJ[0], EJ[1], ej0, ej0l);
      pair_frag_split(EJ[2], EJ[3], ej1, ej1l);
    }
    // (4) dphi(k_j)[d] = (R v_j)[d] + r_d + sum_i E[i][j] phi(q_i)[d];  dk = dphi(k) phi'(k).
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::SM; ++s) {
        const bf16x8 vp = perm_row<GG::UM>(sm.Vs, j_loc, s, g);  // v_j at the permuted m
        acc = mma(jfrag<GG::UD>(sm.Rh, 32 * s, 16 * dt, g, n), vp, acc);
        acc = mma(jfrag<GG::UD>(sm.Rl, 32 * s, 16 * dt, g, n), vp, acc);
      }
      {
        const bf16x8 q0 = jfrag<GG::UD>(sm.Qh, 0, 16 * dt, g, n), q1 = jfrag<GG::UD>(sm.Qh, 32, 16 * dt, g, n);
        acc = mma(q0, ej0, acc);
        acc = mma(q0, ej0l, acc);
        acc = mma(jfrag<GG::UD>(sm.Ql, 0, 16 * dt, g, n), ej0, acc);
        acc = mma(q1, ej1, acc);
        acc = mma(q1, ej1l, acc);
        acc = mma(jfrag<GG::UD>(sm.Ql, 32, 16 * dt, g, n), ej1, acc);
      }
      const f32x4 rr = *reinterpret_cast<const f32x4*>(&sm.rs[16 * dt + 4 * g]);
      const float4 kk = raw4(unit8<GG::UD>(sm.Kr, j_loc, 16 * dt + 4 * g));
      const float o0 = (acc[0] + rr[0]) * dphi_raw(kk.x), o1 = (acc[1] + rr[1]) * dphi_raw(kk.y);
      const float o2 = (acc[2] + rr[2]) * dphi_raw(kk.z), o3 = (acc[3] + rr[3]) * dphi_raw(kk.w);
      if (rowok)
        *reinterpret_cast<u32x2*>(dk + (row0 + j_loc) * D + 16 * dt + 4 * g) = u32x2{cvt_pk(o0, o1), cvt_pk(o2, o3)};
    }
    // (5) R += phi(Q)^T a, r += phi(Q)^T b.
    rstate_update<D, M>(st, sm.Qh, sm.Ql, sm.Ah, sm.Al, sm.Bs, w, n, g);
  }
}

template <int D, int M>
static hipError_t impl(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk, void* dv,
                       int BH, int N, int tblk, int nblk, float* preS, float* preZ, float* inv, float* bw, float* suf,
                       hipStream_t stream) {
  const dim3 grid((unsigned)nblk * (unsigned)BH), block(NT);
  hipLaunchKernelGGL((bwd_q_bf16_kernel<D, M>), grid, block, 0, stream, (const bf16_t*)q, (const bf16_t*)k,
                     (const bf16_t*)v, (const bf16_t*)dO, (bf16_t*)dq, N, tblk, nblk, preS, preZ, inv, bw);
  hipLaunchKernelGGL((bwd_rstate_bf16_kernel<D, M>), grid, block, 0, stream, (const bf16_t*)q, (const bf16_t*)dO, inv,
                     bw, N, tblk, nblk, suf);
  hipError_t e = launch_suffix_scan(suf, BH, nblk, D * M + D, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_kv_bf16_kernel<D, M>), grid, block, 0, stream, (const bf16_t*)q, (const bf16_t*)k,
                     (const bf16_t*)v, (const bf16_t*)dO, inv, bw, (bf16_t*)dk, (bf16_t*)dv, N, tblk, nblk, suf);
  return hipGetLastError();
}

}  // namespace bwdh

hipError_t launch_causal_bwd_bf16(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk,
                                  void* dv, int BH, int N, int D, int M, int tblk, int nblk, float* preS, float* preZ,
                                  float* inv, float* b, float* suf, hipStream_t stream) {
  switch (D * 100 + M) {
    case 3232: return bwdh::impl<32, 32>(q, k, v, dO, dq, dk, dv, BH, N, tblk, nblk, preS, preZ, inv, b, suf, stream);
    case 3264: return bwdh::impl<32, 64>(q, k, v, dO, dq, dk, dv, BH, N, tblk, nblk, preS, preZ, inv, b, suf, stream);
    case 6432: return bwdh::impl<64, 32>(q, k, v, dO, dq, dk, dv, BH, N, tblk, nblk, preS, preZ, inv, b, suf, stream);
    case 6464: return bwdh::impl<64, 64>(q, k, v, dO, dq, dk, dv, BH, N, tblk, nblk, preS, preZ, inv, b, suf, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
