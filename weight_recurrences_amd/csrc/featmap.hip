// Linear attention with the other feature maps the pages name, on gfx950:
// DPFP-nu and the degree-2 polynomial map.
//
// "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器", §3.2.1: a feature map phi of dimension C makes attention
// O(N C M) work, and the degree-2 polynomial kernel has an exact map with
// C = D^2.  News summary of "Linear Transformers Are Secretly Fast Weight
// Programmers", DPFP paragraph: a deterministic, parameter-free map that raises
// the dot-product dimension to 2 nu D.  The maps (the DPFP formula is not
// printed; this is the reading taken):
//   DPFP-nu: r = (relu(x), relu(-x)) in R^{2D},
//            phi(x)_{(n-1) 2D + i} = r_i r_{(i+n) mod 2D},  n = 1..nu;
//   POLY2:   phi(x)_{a D + b} = x_a x_b,  so phi(q).phi(k) = (q.k)^2.
// The attention is eq.(8)-(12) (causal) and eq.(5)-(6) (non-causal) with phi.
//
// Work split.  The C features are cut into slices of FS = 64; a slice of phi is
// itself a feature map, and numerator and denominator are sums over slices.
// The polynomial map is carried on its symmetric pairs a <= b (p2_groups): 2560
// internal features at D = 64 instead of 4096, folded from and expanded to the
// D x D state layout at the boundary.
//   1. fm_state_kernel (head, block of tblk tokens, slice s): the block's state
//      increment dS_s = phi_s(K)^T V, dz_s = column sums of phi_s(K).
//   2. the block scan of the elu + 1 path: exclusive prefix per block (causal)
//      or the total (non-causal), starting from S0.
//   3. fm_out_kernel (head, chunk of 64 queries):
//        num_i = sum_s phi_s(q_i)^T S_s + sum_{j in block, j <= i} sim(q_i, k_j) v_j
//        den_i = sum_s phi_s(q_i)^T z_s + sum_{j in block, j <= i} sim(q_i, k_j)
//      with (S_s, z_s) the prefix state at the block start, o_i = num_i / den_i.
//      DPFP: the block is the chunk (tblk = 64) and sim is summed slice by slice
//      from the features.  POLY2: sim = (q.k)^2 from a D-long dot product, so
//      blocks hold several chunks and fewer prefix states are written.
// Features are formed in fp32 (bf16 inputs are widened on load; outputs are
// rounded to the input dtype).  The state and output products, and DPFP's
// scores, take them as a bf16 head and tail on 16x16x32 bf16 MFMA
// (a.b = ah.bh + ah.bl + al.bh, fp32 accumulation, operands kept to about
// 2^-17 relative); the value products of the scores and the polynomial map's
// (q.k)^2 run on fp32 MFMA (v_mfma_f32_16x16x4_f32).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace la {
namespace fm {

constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr int CH = 64;   // tokens per chunk
constexpr int FS = 64;   // features per slice
constexpr int POLY2 = 4; // template code of the polynomial map; DPFP-nu is coded nu (1..3)

// The polynomial map's features are symmetric (x_a x_b = x_b x_a).  Inside the
// kernels it is carried by the pairs a <= b only, in groups of 16: group (a, h)
// holds b = 16h .. 16h + 15 for h >= a / 16, the key-side features weighted 2
// for b > a, 1 for b = a and 0 for b < a, so that
//   sum_{a <= b, grouped} q_a q_b (w_ab k_a k_b) = (q.k)^2.
// Groups run h-major: group index gi = 8 h (h + 1) + a, a < 16 (h + 1).
template <int D>
constexpr int p2_groups() {
  return 8 * (D / 16) * (D / 16 + 1);
}

// Internal feature dimension (what the kernels and the block records carry).
template <int FM, int D>
constexpr int fdim() {
  return FM == POLY2 ? 16 * p2_groups<D>() : 2 * FM * D;
}

// (a, h) of polynomial group gi (uniform; D <= 64 gives h <= 3).
__device__ __forceinline__ void p2_group(int gi, int& a, int& h) {
  h = gi >= 96 ? 3 : (gi >= 48 ? 2 : (gi >= 16 ? 1 : 0));
  a = gi - 8 * h * (h + 1);
}

// Rows [0, nv) of a row-major [.][W] tensor starting at src, widened to float
// into LDS (row stride DS floats); rows nv..63 become zeros.  The loads carry
// no condition (rows past nv re-read row nv - 1 and are replaced by zeros): a
// conditional load becomes a branch at which the compiler waits for every load
// in flight, which would turn the loads into one round trip each.
template <typename T, int W>
__device__ __forceinline__ void fetch_rows(float4 (&x)[CH * W / 4 / NT], const T* src, int nv, int tid) {
#pragma unroll
  for (int u = 0; u < CH * W / 4 / NT; ++u) {
    const int e = (u * NT + tid) * 4, r = e / W, c = e % W;
    x[u] = load4<T>(src + (size_t)min(r, nv - 1) * W + c);
  }
}
template <int W, int DS>
__device__ __forceinline__ void put_rows(float* dst, const float4 (&x)[CH * W / 4 / NT], int nv, int tid) {
#pragma unroll
  for (int u = 0; u < CH * W / 4 / NT; ++u) {
    const int e = (u * NT + tid) * 4, r = e / W, c = e % W;
    *reinterpret_cast<float4*>(dst + r * DS + c) = r < nv ? x[u] : float4{0.f, 0.f, 0.f, 0.f};
  }
}

template <typename T, int W, int DS>
__device__ __forceinline__ void load_rows(float* dst, const T* src, int nv, int tid) {
  constexpr int G = CH * W / 4;  // groups of four elements
  static_assert(G % NT == 0, "whole groups per thread");
  float4 x[G / NT];
  if (nv > 0) {
#pragma unroll
    for (int u = 0; u < G / NT; ++u) {
      const int e = (u * NT + tid) * 4, r = e / W, c = e % W;
      x[u] = load4<T>(src + (size_t)min(r, nv - 1) * W + c);
    }
  }
#pragma unroll
  for (int u = 0; u < G / NT; ++u) {
    const int e = (u * NT + tid) * 4, r = e / W, c = e % W;
    *reinterpret_cast<float4*>(dst + r * DS + c) = r < nv ? x[u] : float4{0.f, 0.f, 0.f, 0.f};
  }
}

// Rows [0, nv) of a row-major [.][D] tensor as r = (relu(x), relu(-x)) in LDS
// (row stride DS >= 2 D floats); rows nv..63 become zeros.  A DPFP feature is
// then the product r_i r_j of two stored values.  Loads as in load_rows.
template <typename T, int D, int DS>
__device__ __forceinline__ void load_relu_rows(float* dst, const T* src, int nv, int tid) {
  constexpr int G = CH * D / 4;
  static_assert(G % NT == 0, "whole groups per thread");
  float4 x[G / NT];
  if (nv > 0) {
#pragma unroll
    for (int u = 0; u < G / NT; ++u) {
      const int e = (u * NT + tid) * 4, r = e / D, c = e % D;
      x[u] = load4<T>(src + (size_t)min(r, nv - 1) * D + c);
    }
  }
#pragma unroll
  for (int u = 0; u < G / NT; ++u) {
    const int e = (u * NT + tid) * 4, r = e / D, c = e % D;
    const float4 p = r < nv ? x[u] : float4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<float4*>(dst + r * DS + c) =
        float4{fmaxf(p.x, 0.f), fmaxf(p.y, 0.f), fmaxf(p.z, 0.f), fmaxf(p.w, 0.f)};
    *reinterpret_cast<float4*>(dst + r * DS + D + c) =
        float4{fmaxf(-p.x, 0.f), fmaxf(-p.y, 0.f), fmaxf(-p.z, 0.f), fmaxf(-p.w, 0.f)};
  }
}

// Eight floats as a bf16 head and tail (x = h + l to about 2^-17 relative).
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& h, bf16x8& l) {
  u32x4 hv, lv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hv[i] = cvt_pk(x[2 * i], x[2 * i + 1]);
    lv[i] = cvt_pk(x[2 * i] - lo_of(hv[i]), x[2 * i + 1] - hi_of(hv[i]));
  }
  h = as_bf16x8(hv);
  l = as_bf16x8(lv);
}

// ---- 1. block state increments ---------------------------------------------
// grid: BH * nblk * (NS / SG), blockIdx.x = (bh * nblk + blk) * (NS / SG) + sg;
// the workgroup covers slices sg*SG .. sg*SG + SG - 1 of one block, so the
// block's keys and values are read once for SG slices.
// agg [BH * NS][nblk][FS][M], aggz [BH * NS][nblk][FS].
// Tile: rows = the 16 features 16w.. of the slice, columns = values, k-slot =
// token (bf16 16x16x32 MFMA on head/tail operands); features are formed from
// the raw key rows as the operand is read, and the lane's operands also give
// its share of z.
// The largest divisor of NS up to 4: more slices per workgroup read the rows
// fewer times but hold more accumulators (the polynomial map, 40 slices: 888 us
// per call with groups of 8, 814 with 4, 901 with 2).
template <int NS>
constexpr int slice_group() {
  int g = NS < 4 ? NS : 4;
  while (NS % g) --g;
  return g;
}

template <typename T, int D, int M, int FM>
__global__ __launch_bounds__(NT, 2) void fm_state_kernel(const T* __restrict__ k, const T* __restrict__ v, int N,
                                                      int tblk, int nblk, float* __restrict__ agg,
                                                      float* __restrict__ aggz) {
  constexpr int NS = fdim<FM, D>() / FS, SG = slice_group<NS>(), TM = M / 16;
  static_assert(NS % SG == 0, "whole slice groups");
  // Row strides of 16 banks: the four k-slot groups g read four different rows.
  // DPFP keeps r = (relu(k), relu(-k)) per key row (2 D floats), the polynomial
  // map the raw row.
  constexpr int KS = (FM == POLY2 ? D : 2 * D) + 16, VS = M + 16;
  __shared__ __attribute__((aligned(16))) float Kr[CH * KS];
  __shared__ __attribute__((aligned(16))) float Vs[CH * VS];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform: its tests are scalar branches
  const int sg = blockIdx.x % (NS / SG), rest = blockIdx.x / (NS / SG), blk = rest % nblk, bh = rest / nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const T* kh = k + (size_t)bh * N * D;
  const T* vh = v + (size_t)bh * N * M;
  f32x4 acc[SG][TM];
  float zp[SG];
  int pa[SG], pb[SG];  // polynomial: the lane's pair (a, b) per slice of the group
  float pw[SG];        // and its weight
#pragma unroll
  for (int j = 0; j < SG; ++j) {
    zp[j] = 0.f;
#pragma unroll
    for (int vb = 0; vb < TM; ++vb) acc[j][vb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FM == POLY2) {  // wave w holds group 4 s + w of slice s
      int a, h;
      p2_group(4 * (sg * SG + j) + w, a, h);
      pa[j] = a;
      pb[j] = 16 * h + n;
      pw[j] = pb[j] > a ? 2.f : (pb[j] == a ? 1.f : 0.f);
    }
  }
  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    __syncthreads();  // the previous chunk's readers are done
    if constexpr (FM == POLY2) {
      load_rows<T, D, KS>(Kr, kh + (size_t)c0 * D, nv, tid);
    } else {
      load_relu_rows<T, D, KS>(Kr, kh + (size_t)c0 * D, nv, tid);
    }
    load_rows<T, M, VS>(Vs, vh + (size_t)c0 * M, nv, tid);
    __syncthreads();
    // 32-token slabs on bf16 MFMA with head/tail operands (a b = ah bh + ah bl +
    // al bh, float32 accumulation): k-slot 8g + e of slab s is token 32 s + 4 e + g,
    // so that the four lane groups read four consecutive rows (distinct banks).
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      bf16x8 bvh[TM], bvl[TM];
#pragma unroll
      for (int vb = 0; vb < TM; ++vb) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = Vs[(32 * s + 4 * e + g) * VS + 16 * vb + n];
        split_bf16x8(x, bvh[vb], bvl[vb]);
      }
#pragma unroll
      for (int j = 0; j < SG; ++j) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float* kr = Kr + (32 * s + 4 * e + g) * KS;
          if constexpr (FM == POLY2) {
            a[e] = pw[j] * kr[pa[j]] * kr[pb[j]];
          } else {  // feature c = r_i r_{(i + n) mod 2D}, i = c mod 2D, n = c / 2D + 1
            const int c = (sg * SG + j) * FS + 16 * w + n, i = c % (2 * D);
            a[e] = kr[i] * kr[(i + c / (2 * D) + 1) % (2 * D)];
          }
          zp[j] += a[e];
        }
        bf16x8 ah, al;
        split_bf16x8(a, ah, al);
#pragma unroll
        for (int vb = 0; vb < TM; ++vb) {
          acc[j][vb] = mma(ah, bvh[vb], acc[j][vb]);
          acc[j][vb] = mma(ah, bvl[vb], acc[j][vb]);
          acc[j][vb] = mma(al, bvh[vb], acc[j][vb]);
        }
        // One slice at a time: the features of later slices are not formed early
        // (which would keep them all live).
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // acc[j][vb]: lane (n, g) holds features 16w + 4g + i of value column 16 vb + n.
#pragma unroll
  for (int j = 0; j < SG; ++j) {
    const size_t rec = (size_t)(bh * NS + sg * SG + j) * nblk + blk;
    float* S = agg + rec * FS * M;
#pragma unroll
    for (int vb = 0; vb < TM; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[(16 * w + 4 * g + i) * M + 16 * vb + n] = acc[j][vb][i];
    float z = zp[j];
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    if (g == 0) aggz[rec * FS + 16 * w + n] = z;
  }
}

// ---- 3. outputs --------------------------------------------------------------
template <int D, int M, bool KF>
struct OutSmem {
  static constexpr int XS = D + 4, VS = M + 4;
  float Qr[CH * XS];  // raw queries of the chunk
  float Kr[CH * XS];  // raw keys of the current key chunk
  union {             // the state slices during the slice loop, the values after it
    float Vs[CH * VS];
    struct {
      bf16_t Sh[FS * M];  // prefix state slice S_s [FS][M] as a bf16 head and tail, row-major swizzled
      bf16_t Sl[FS * M];
      bf16_t Kh[KF ? CH * FS : 8];  // DPFP: the slice's key features [key][FS], head and tail, swizzled
      bf16_t Kl[KF ? CH * FS : 8];
    } st;
  };
  float zs[FS];  // prefix z slice
};

// Four DPFP features base + f0 + r (r < 4) of a raw row x from two 16-byte LDS
// reads: r_i r_{i + ORD} with i = base + f0 + r (base a multiple of D, f0 of 4,
// ORD in 1..3).  A lane's four consecutive elements in one read keep the rows'
// accesses free of bank conflicts (four-byte reads of a column group across
// rows collide).  Per call against four-byte reads (same-box A/B): DPFP-1
// 101.4 -> 96.6 us, DPFP-2 169.5 -> 159.3 us.
template <int D, int ORD>
__device__ __forceinline__ void dpfp4(const float* x, int base, int f0, float (&out)[4]) {
  static_assert(ORD >= 1 && ORD <= 3, "partner shift 1..3");
  const float4 a = *reinterpret_cast<const float4*>(x + (f0 & (D - 1)));
  const float4 b = *reinterpret_cast<const float4*>(x + ((f0 + 4) & (D - 1)));
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const bool negi = ((base + f0) & D) != 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float xi = v[r], xj = v[r + ORD];
    const bool negj = ((base + f0 + r + ORD) & D) != 0;
    out[r] = fmaxf(negi ? -xi : xi, 0.f) * fmaxf(negj ? -xj : xj, 0.f);
  }
}

// grid: BH * nqc, blockIdx.x = bh * nqc + qc (nqc = ceil(N / 64) query chunks).
// pre/prez: causal, the exclusive block prefixes [BH * NS][nblk][FS][M] / [FS];
// non-causal, the totals [BH * NS][FS][M] / [FS].
// Features are formed from the raw rows as MFMA operands are read.  The tiles
// are transposed, rows = values or keys and columns = the wave's 16 queries,
// so a score tile is already the B operand of the value product.
template <typename T, int D, int M, int FM>
__global__ __launch_bounds__(NT) void fm_out_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, T* __restrict__ o, int N, int tblk,
                                                    int nblk, const float* __restrict__ pre,
                                                    const float* __restrict__ prez, int causal, int BHN) {
  using SM = OutSmem<D, M, FM != POLY2>;
  constexpr int NS = fdim<FM, D>() / FS, TM = M / 16;
  constexpr int XS = SM::XS, VS = SM::VS;
  constexpr int PF = FS * M / 4 / NT;  // float4 groups of a state slice per thread
  __shared__ __attribute__((aligned(16))) SM sm;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform: its tests are scalar branches
  const int nqc = (N + CH - 1) / CH;
  // Workgroup ids go round-robin over the 8 XCDs.  With G = tblk / 64 query
  // chunks per block (causal), the ids are remapped so that G consecutive chunks,
  // which read the same prefix state, run on one XCD and share its L2; the grid
  // is padded to whole groups of 8 G and the padding exits at once.
  const int G = causal ? tblk / CH : 1;
  int L = blockIdx.x;
  if (G > 1) {
    const int xcd = L & 7, kx = L >> 3;
    L = ((kx / G) * 8 + xcd) * G + kx % G;
  }
  if (L >= BHN) return;
  const int qc = L % nqc, bh = L / nqc;
  const int q0 = qc * CH, nq = min(CH, N - q0);
  const int blk = causal ? q0 / tblk : 0, npre = causal ? nblk : 1;
  const T* qh = q + (size_t)bh * N * D;
  const T* kh = k + (size_t)bh * N * D;
  const T* vh = v + (size_t)bh * N * M;
  const float* Sb = pre + ((size_t)bh * NS * npre + blk) * FS * M;  // slice s at + s * npre * FS * M
  const float* zb = prez + ((size_t)bh * NS * npre + blk) * FS;
  const size_t sstride = (size_t)npre * FS * M;
  const bool intra_dpfp = FM != POLY2 && causal;

  // The first state slice is requested before the raw rows, so both are in flight.
  f32x4 pf[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) pf[u] = *reinterpret_cast<const f32x4*>(Sb + (u * NT + tid) * 4);
  float pz = zb[min(tid, FS - 1)];  // lanes tid >= FS never store theirs
  load_rows<T, D, XS>(sm.Qr, qh + (size_t)q0 * D, nq, tid);
  if (intra_dpfp) load_rows<T, D, XS>(sm.Kr, kh + (size_t)q0 * D, nq, tid);  // the block is this chunk
  float4 vpre[CH * M / 4 / NT];
  if constexpr (FM != POLY2) fetch_rows<T, M>(vpre, vh + (size_t)q0 * M, intra_dpfp ? nq : 1, tid);
  f32x4 num[TM];  // num^T tiles: lane (n, g) holds values 16 vb + 4g + i of query 16w + n
#pragma unroll
  for (int vb = 0; vb < TM; ++vb) num[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 at[4];  // DPFP: score tiles A^T (keys 16 kb.. x the wave's queries), summed over slices
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) at[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;  // partial over the features (or keys) this lane's k-slots cover
  const float* qrow = sm.Qr + (16 * w + n) * XS;

  // The slice loop is compiled once per wave index W, so the key tiles a wave
  // scores (kb <= W) are known at compile time and its accumulators stay in place.
  auto slices = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    // One slice s of the features.  ORD is a DPFP slice's partner shift (the
    // order n of its features r_i r_{i+n}), a constant in each copy of the body.
    auto slice = [&](const int s, auto oc) {
      constexpr int ORD = decltype(oc)::value;
      __syncthreads();  // raw rows stored; the previous slice's readers are done
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int e = (u * NT + tid) * 4, f = e / M, c = e % M;
        const f32x4 x = pf[u];
        const uint32_t h0 = cvt_pk(x[0], x[1]), h1 = cvt_pk(x[2], x[3]);
        unit8<M / 8>(sm.st.Sh, f, c) = u32x2{h0, h1};
        unit8<M / 8>(sm.st.Sl, f, c) =
            u32x2{cvt_pk(x[0] - lo_of(h0), x[1] - hi_of(h0)), cvt_pk(x[2] - lo_of(h1), x[3] - hi_of(h1))};
      }
      if (tid < FS) sm.zs[tid] = pz;
      const int base = (s * FS) & (2 * D - 1);
      constexpr int order = ORD;
      if (FM != POLY2 && intra_dpfp) {  // the slice's features of the chunk's keys, formed once for all waves
        const int r = tid >> 2, f0 = 16 * (tid & 3);
        const float* krow = sm.Kr + r * XS;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float kv[8], k0[4], k1[4];
          dpfp4<D, order>(krow, base, f0 + 8 * hf, k0);
          dpfp4<D, order>(krow, base, f0 + 8 * hf + 4, k1);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kv[r] = k0[r];
            kv[4 + r] = k1[r];
          }
          bf16x8 kh8, kl8;
          split_bf16x8(kv, kh8, kl8);
          unit16<FS / 8>(sm.st.Kh, r, f0 + 8 * hf) = __builtin_bit_cast(u32x4, kh8);
          unit16<FS / 8>(sm.st.Kl, r, f0 + 8 * hf) = __builtin_bit_cast(u32x4, kl8);
        }
      }
      {  // next slice in flight during this one (the last slice re-reads itself; unconditional loads, as in load_rows)
        const int sn = min(s + 1, NS - 1);
#pragma unroll
        for (int u = 0; u < PF; ++u)
          pf[u] = *reinterpret_cast<const f32x4*>(Sb + (size_t)sn * sstride + (u * NT + tid) * 4);
        pz = zb[(size_t)sn * npre * FS + min(tid, FS - 1)];
      }
      __syncthreads();
      // Inter-block part: num^T += S_s^T phi_s(Q)^T, den += phi_s(Q) z_s; for DPFP
      // also the slice's share of the chunk's scores.  bf16 16x16x32 MFMA on head/
      // tail operands over 32-feature slabs: k-slot e = 4h + r of lane group g is
      // feature 32 s2 + 16 h + 4 g + r, the order in which the transposed reads of
      // the state rows deliver them.
      float pqa[4];  // polynomial: q_a of the slice's four groups, and their b offset 16 h
      int pb0[4];
      if constexpr (FM == POLY2) {
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
          int a, h;
          p2_group(4 * s + tg, a, h);
          pqa[tg] = qrow[a];
          pb0[tg] = 16 * h;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < FS / 32; ++s2) {
        float qv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // features f0 + r, f0 = 32 s2 + 16 h + 4 g: 16-byte reads
          const int f0 = 32 * s2 + 16 * h + 4 * g;
          float q4[4];
          if constexpr (FM == POLY2) {
            const float4 qb = *reinterpret_cast<const float4*>(qrow + pb0[2 * s2 + h] + 4 * g);
            const float qa = pqa[2 * s2 + h];
            q4[0] = qa * qb.x;
            q4[1] = qa * qb.y;
            q4[2] = qa * qb.z;
            q4[3] = qa * qb.w;
          } else {
            dpfp4<D, order>(qrow, base, f0, q4);
          }
          const float4 zf = *reinterpret_cast<const float4*>(&sm.zs[f0]);
          den += q4[0] * zf.x + q4[1] * zf.y + q4[2] * zf.z + q4[3] * zf.w;
#pragma unroll
          for (int r = 0; r < 4; ++r) qv[4 * h + r] = q4[r];
        }
        bf16x8 qh8, ql8;
        split_bf16x8(qv, qh8, ql8);
#pragma unroll
        for (int vb = 0; vb < TM; ++vb) {
          const bf16x8 ah = jfrag<M / 8>(sm.st.Sh, 32 * s2, 16 * vb, g, n);
          const bf16x8 al = jfrag<M / 8>(sm.st.Sl, 32 * s2, 16 * vb, g, n);
          num[vb] = mma(ah, qh8, num[vb]);
          num[vb] = mma(ah, ql8, num[vb]);
          num[vb] = mma(al, qh8, num[vb]);
        }
        if (intra_dpfp) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            if (kb <= W) {  // key rows 16 kb + n at the k-slots of the query features
              const u32x2 h0 = unit8<FS / 8>(sm.st.Kh, 16 * kb + n, 32 * s2 + 4 * g);
              const u32x2 h1 = unit8<FS / 8>(sm.st.Kh, 16 * kb + n, 32 * s2 + 16 + 4 * g);
              const u32x2 l0 = unit8<FS / 8>(sm.st.Kl, 16 * kb + n, 32 * s2 + 4 * g);
              const u32x2 l1 = unit8<FS / 8>(sm.st.Kl, 16 * kb + n, 32 * s2 + 16 + 4 * g);
              const bf16x8 kh8 = as_bf16x8(u32x4{h0[0], h0[1], h1[0], h1[1]});
              const bf16x8 kl8 = as_bf16x8(u32x4{l0[0], l0[1], l1[0], l1[1]});
              at[kb] = mma(kh8, qh8, at[kb]);
              at[kb] = mma(kh8, ql8, at[kb]);
              at[kb] = mma(kl8, qh8, at[kb]);
            }
          }
        }
      }
    };
    if constexpr (FM == POLY2) {
      for (int s = 0; s < NS; ++s) slice(s, std::integral_constant<int, 1>{});
    } else {  // slices in feature order, which groups them by shift: NS / FM per shift
      constexpr int SPO = NS / FM;
      for (int hs = 0; hs < SPO; ++hs) slice(hs, std::integral_constant<int, 1>{});
      if constexpr (FM >= 2)
        for (int hs = 0; hs < SPO; ++hs) slice(SPO + hs, std::integral_constant<int, 2>{});
      if constexpr (FM >= 3)
        for (int hs = 0; hs < SPO; ++hs) slice(2 * SPO + hs, std::integral_constant<int, 3>{});
    }

    if (intra_dpfp) {
      // The values replace the state slices in LDS.
      __syncthreads();
      put_rows<M, VS>(sm.Vs, vpre, nq, tid);
      __syncthreads();
      // Keys after the query are masked; num^T += V^T A^T, den += column sums of A^T.
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f32x4 a = at[kb];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb == W && 4 * g + i > n) a[i] = 0.f;
        if (kb <= W) {
          den += a[0] + a[1] + a[2] + a[3];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int vb = 0; vb < TM; ++vb)
              num[vb] = mma(sm.Vs[(16 * kb + 4 * g + i) * VS + 16 * vb + n], a[i], num[vb]);
        }
      }
    }
  };
  if constexpr (FM == POLY2) {
    slices(std::integral_constant<int, 3>{});  // no DPFP scores: one copy
  } else {
    switch (w) {
      case 0: slices(std::integral_constant<int, 0>{}); break;
      case 1: slices(std::integral_constant<int, 1>{}); break;
      case 2: slices(std::integral_constant<int, 2>{}); break;
      default: slices(std::integral_constant<int, 3>{}); break;
    }
  }

  if constexpr (FM == POLY2) {
    // Intra-block part: sim = (q.k)^2 for the block's keys up to this chunk.
    if (causal) {
      // Each key chunk's rows are fetched into registers while the previous one
      // is scored (the last chunk re-reads itself: unconditional loads).
      float4 kpf[CH * D / 4 / NT], vpf[CH * M / 4 / NT];
      fetch_rows<T, D>(kpf, kh + (size_t)blk * tblk * D, min(CH, N - blk * tblk), tid);
      fetch_rows<T, M>(vpf, vh + (size_t)blk * tblk * M, min(CH, N - blk * tblk), tid);
      for (int kc0 = blk * tblk; kc0 <= q0; kc0 += CH) {
        const int nk = min(CH, N - kc0);
        __syncthreads();  // the previous key chunk's readers are done
        put_rows<D, XS>(sm.Kr, kpf, nk, tid);
        put_rows<M, VS>(sm.Vs, vpf, nk, tid);
        __syncthreads();
        {
          const int kn = min(kc0 + CH, q0);
          fetch_rows<T, D>(kpf, kh + (size_t)kn * D, min(CH, N - kn), tid);
          fetch_rows<T, M>(vpf, vh + (size_t)kn * M, min(CH, N - kn), tid);
        }
        // The four key tiles' scores run as four interleaved chains; on the
        // diagonal chunk the tiles past the wave's queries are masked to zero
        // (no branch around the products).
        const bool diag = kc0 == q0;
        f32x4 a4[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) a4[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < D / 4; ++t) {
          const float qx = qrow[4 * t + g];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) a4[kb] = mma(sm.Kr[(16 * kb + n) * XS + 4 * t + g], qx, a4[kb]);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          f32x4 a = a4[kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] *= a[i];
            if (diag && (kb > w || (kb == w && 4 * g + i > n))) a[i] = 0.f;
          }
          den += a[0] + a[1] + a[2] + a[3];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int vb = 0; vb < TM; ++vb)
              num[vb] = mma(sm.Vs[(16 * kb + 4 * g + i) * VS + 16 * vb + n], a[i], num[vb]);
        }
      }
    }
  }

  den += __shfl_xor(den, 16);
  den += __shfl_xor(den, 32);
  if (16 * w + n < nq) {
    const float rd = __builtin_amdgcn_rcpf(den);  // 1 ulp; 0/0 rows stay NaN (0 * inf)
    T* orow = o + ((size_t)bh * N + q0 + 16 * w + n) * M + 4 * g;
#pragma unroll
    for (int vb = 0; vb < TM; ++vb)
      store4<T>(orow + 16 * vb, float4{num[vb][0] * rd, num[vb][1] * rd, num[vb][2] * rd, num[vb][3] * rd});
  }
}

// Polynomial map, full state [BH][D*D][M] (+ z [BH][D*D]) -> grouped state
// [BH][CI][M] (+ [BH][CI]): pair (a, b), a < b, takes S_ab + S_ba; a = b takes
// S_aa; the zero-weight slots (b < a inside a group) are 0.  Then
// sum_{grouped} q_a q_b S'_ab = sum_{a,b} q_a q_b S_ab for any S.
// grid: ceil(BH * CI * (M + 1) / NT); element e = (bh * CI + c) * (M + 1) + m, m = M is z.
template <int D, int M>
__global__ __launch_bounds__(NT) void p2_fold_kernel(const float* __restrict__ S, const float* __restrict__ z,
                                                     float* __restrict__ Sf, float* __restrict__ zf, long long n) {
  constexpr int CI = fdim<POLY2, D>();
  const long long e = (long long)blockIdx.x * NT + threadIdx.x;
  if (e >= n) return;
  const int m = (int)(e % (M + 1));
  const long long bc = e / (M + 1);
  const int c = (int)(bc % CI);
  const long long bh = bc / CI;
  int a, h;
  p2_group(c >> 4, a, h);
  const int b = 16 * h + (c & 15);
  float r = 0.f;
  if (m < M) {
    const float* Sh = S + bh * D * D * M;
    if (b > a) r = Sh[(a * D + b) * M + m] + Sh[(b * D + a) * M + m];
    else if (b == a) r = Sh[(a * D + a) * M + m];
    Sf[bc * M + m] = r;
  } else {
    const float* zh = z + bh * D * D;
    if (b > a) r = zh[a * D + b] + zh[b * D + a];
    else if (b == a) r = zh[a * D + a];
    zf[bc] = r;
  }
}

// Grouped state back to the full layout: S_out_ab = S0_ab + (S'_tot - S'_0) at
// the pair (min, max), divided by its weight (2 off the diagonal).  S0 and the
// folded S'_0 may be NULL (zero start).  Every output element reads only its
// own S0 element, so S_out may be S0.
// grid: ceil(BH * D * D * (M + 1) / NT); element e = (bh * D * D + a * D + b) * (M + 1) + m.
template <int D, int M>
__global__ __launch_bounds__(NT) void p2_expand_kernel(const float* S0, const float* z0,
                                                       const float* __restrict__ Sf0, const float* __restrict__ zf0,
                                                       const float* __restrict__ Stot, const float* __restrict__ ztot,
                                                       float* S_out, float* z_out, long long n) {
  constexpr int CI = fdim<POLY2, D>();
  const long long e = (long long)blockIdx.x * NT + threadIdx.x;
  if (e >= n) return;
  const int m = (int)(e % (M + 1));
  const long long bab = e / (M + 1);
  const int ab = (int)(bab % (D * D));
  const long long bh = bab / (D * D);
  const int a = ab / D, b = ab % D, lo = a < b ? a : b, hi = a < b ? b : a, h = hi >> 4;
  const long long c = bh * CI + 16 * (8 * h * (h + 1) + lo) + (hi & 15);
  const float inv_w = lo < hi ? 0.5f : 1.f;
  if (m < M) {
    const float d = Stot[c * M + m] - (Sf0 ? Sf0[c * M + m] : 0.f);
    S_out[bab * M + m] = (S0 ? S0[bab * M + m] : 0.f) + d * inv_w;
  } else {
    const float d = ztot[c] - (zf0 ? zf0[c] : 0.f);
    z_out[bab] = (z0 ? z0[bab] : 0.f) + d * inv_w;
  }
}

// Tokens per block: the chunk for DPFP (its intra-block similarity is built from
// the features, slice by slice); 512 for the polynomial map (intra-block
// similarity from D-long dot products, fewer prefix states: per call at
// B=4 H=8 N=4096 D=64, 826 us with 128, 611 with 256, 588 with 512 and 638
// with 1024, where the intra-block work outgrows the records it saves).
template <int FM>
static int block_tokens(int N) {
  if constexpr (FM != POLY2) {
    return CH;
  } else {
    const int cap = ((N + CH - 1) / CH) * CH;
    return cap < 512 ? (cap > 0 ? cap : CH) : 512;
  }
}

template <int FM>
static size_t ws_bytes_t(int BH, int N, int D, int M) {
  const int C = FM == POLY2 ? (D == 64 ? fdim<POLY2, 64>() : fdim<POLY2, 32>()) : 2 * FM * D;
  const int NS = C / FS;
  const int tblk = block_tokens<FM>(N);
  const size_t nblk = (size_t)((N + tblk - 1) / tblk);
  // block records, the totals, and (polynomial map) the folded initial state
  const size_t totals = (size_t)BH * C * (M + 1);
  return ((size_t)BH * NS * nblk * (FS * M + FS) + totals + (FM == POLY2 ? totals : 0)) * sizeof(float);
}

template <typename T, int D, int M, int FM>
static hipError_t impl(const void* q, const void* k, const void* v, void* o, int BH, int N, int causal,
                       const float* S0, const float* z0, float* S_out, float* z_out, void* ws, hipStream_t stream) {
  constexpr int C = fdim<FM, D>(), NS = C / FS, CX = FM == POLY2 ? D * D : C;  // internal, external
  static_assert(C % FS == 0, "whole feature slices");
  if (N == 0) {
    if (S_out) return launch_state_copy(S0, z0, S_out, z_out, (long long)BH * CX * M, (long long)BH * CX, stream);
    return hipSuccess;
  }
  const int tblk = block_tokens<FM>(N);
  const int nblk = (N + tblk - 1) / tblk;
  float* agg = (float*)ws;
  float* aggz = agg + (size_t)BH * NS * nblk * FS * M;
  float* Stot = aggz + (size_t)BH * NS * nblk * FS;
  float* ztot = Stot + (size_t)BH * C * M;
  float* Sf0 = ztot + (size_t)BH * C;  // polynomial map: S0 folded onto the grouped pairs
  float* zf0 = Sf0 + (size_t)BH * C * M;
  hipLaunchKernelGGL((fm_state_kernel<T, D, M, FM>),
                     dim3((unsigned)BH * (unsigned)nblk * (unsigned)(NS / slice_group<NS>())), dim3(NT),
                     0, stream, (const T*)k, (const T*)v, N, tblk, nblk, agg, aggz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (FM == POLY2) {
    // The scan runs on the grouped pairs: S0 is folded onto them first, and the
    // grouped total is expanded to the full D x D layout for S_out.
    if (S0) {
      const long long n = (long long)BH * C * (M + 1);
      hipLaunchKernelGGL((p2_fold_kernel<D, M>), dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, stream, S0, z0,
                         Sf0, zf0, n);
    }
    const bool tot = S_out || !causal;
    e = launch_state_scan(agg, aggz, BH * NS, nblk, FS * M, FS, S0 ? Sf0 : nullptr, S0 ? zf0 : nullptr,
                          tot ? Stot : nullptr, tot ? ztot : nullptr, causal, stream);
    if (e != hipSuccess) return e;
    if (S_out) {
      const long long n = (long long)BH * D * D * (M + 1);
      hipLaunchKernelGGL((p2_expand_kernel<D, M>), dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, stream, S0,
                         z0, S0 ? Sf0 : nullptr, S0 ? zf0 : nullptr, Stot, ztot, S_out, z_out, n);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    float* St = S_out ? S_out : (causal ? nullptr : Stot);
    float* zt = S_out ? z_out : (causal ? nullptr : ztot);
    e = launch_state_scan(agg, aggz, BH * NS, nblk, FS * M, FS, S0, z0, St, zt, causal, stream);
    if (e != hipSuccess) return e;
    Stot = St;
    ztot = zt;
  }
  if (!o) return hipSuccess;
  const int nqc = (N + CH - 1) / CH;
  const long long BHN = (long long)BH * nqc;              // query chunks
  const long long grp = causal && tblk > CH ? 8LL * (tblk / CH) : 1;
  const long long nwg = (BHN + grp - 1) / grp * grp;      // padded to whole XCD groups
  hipLaunchKernelGGL((fm_out_kernel<T, D, M, FM>), dim3((unsigned)nwg), dim3(NT), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (T*)o, N, tblk, nblk, causal ? agg : Stot, causal ? aggz : ztot, causal,
                     (int)BHN);
  return hipGetLastError();
}

template <typename T, int D, int M>
static hipError_t fm_entry(int map, const void* q, const void* k, const void* v, void* o, int BH, int N, int causal,
                           const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                           hipStream_t stream) {
  switch (map) {
    case 1: return impl<T, D, M, 1>(q, k, v, o, BH, N, causal, S0, z0, S_out, z_out, ws, stream);
    case 2: return impl<T, D, M, 2>(q, k, v, o, BH, N, causal, S0, z0, S_out, z_out, ws, stream);
    case 3: return impl<T, D, M, 3>(q, k, v, o, BH, N, causal, S0, z0, S_out, z_out, ws, stream);
    case POLY2: return impl<T, D, M, POLY2>(q, k, v, o, BH, N, causal, S0, z0, S_out, z_out, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fm

// map: 1..3 = DPFP-nu, 4 = degree-2 polynomial.
int featmap_dim(int map, int D) { return map == fm::POLY2 ? D * D : (map >= 1 && map <= 3 ? 2 * map * D : 0); }

size_t featmap_ws_bytes(int map, int BH, int N, int D, int M) {
  if (BH <= 0 || N <= 0) return 0;
  switch (map) {
    case 1: return fm::ws_bytes_t<1>(BH, N, D, M);
    case 2: return fm::ws_bytes_t<2>(BH, N, D, M);
    case 3: return fm::ws_bytes_t<3>(BH, N, D, M);
    case fm::POLY2: return fm::ws_bytes_t<fm::POLY2>(BH, N, D, M);
    default: return 0;
  }
}

hipError_t launch_featmap(int map, const void* q, const void* k, const void* v, void* o, int BH, int N, int D,
                          int M, int bf16, int causal, const float* S0, const float* z0, float* S_out, float* z_out,
                          void* ws, hipStream_t stream) {
  if (bf16) {
    LA_DISPATCH_DM(fm::fm_entry, bf16_t, map, q, k, v, o, BH, N, causal, S0, z0, S_out, z_out, ws, stream)
  } else {
    LA_DISPATCH_DM(fm::fm_entry, float, map, q, k, v, o, BH, N, causal, S0, z0, S_out, z_out, ws, stream)
  }
}

}  // namespace la
