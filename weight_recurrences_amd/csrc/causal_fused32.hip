// Single-pass causal linear attention for float32 inputs on gfx950 (MI355X).
//
// Method: "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器", §3.3 eq.(9)-(12): o_i = phi(q_i)^T S_i / phi(q_i)^T z_i with the
// prefix states S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j).
//
// One workgroup owns a block of TB = 256 tokens (four chunks of 64) of one
// (batch, head):
//   pass 1   the block's increment dS = phi(K)^T V, dz = colsum phi(K), chunk by
//            chunk in the order 1, 2, 3, 0, published for the later blocks of
//            the head; chunk 0's tiles are then still in LDS, and its outputs
//            within the block are formed while the increment's stores drain;
//   phase 2  decoupled look-back (lookback.hpp): the exclusive prefix P of the
//            block from the published states of earlier blocks;
//   pass 2   the outputs from the running prefix R_c (P plus the chunks of the
//            block before c): for query i of chunk c
//              num_i = phi(q_i)^T R_c + sum_{j in c, j<=i} (phi(q_i).phi(k_j)) v_j,
//              den_i likewise with z; o_i = num_i / den_i; then R_{c+1} = R_c + dS_c
//            (chunk 0 only adds phi(q_i)^T P to what pass 1 left).
// Pass 2 reads chunks 1..3 of the block's keys and values a second time; pass 1
// reads them with ordinary loads, so the second reads are mostly served by the
// caches (the Infinity Cache holds them between the passes).  Holding the partial outputs of four chunks across the look-back,
// as the bf16 kernel does, would take 128 more registers here (float32 operands
// are a head and a tail), and 64-token blocks instead make the look-back fold
// about ten float32 states per block.
//
// Every product is a bf16 16x16x32 MFMA on head/tail operands (x = h + l to
// about 2^-17 relative), a b = ah bh + ah bl + al bh with float32 accumulation
// (the tail x tail term, about 2^-16 of a product, is dropped), so outputs and
// states carry float32-level error.  The published states are float32.
//
// Operand layouts (lane l = 16 g + n of a 64-lane wavefront) as in the bf16
// kernel: d-contraction slots d = 32 s + 8 g + e of slab s; j-contraction slots
// j = 32 s + 16 h + 4 g + r (e = 4 h + r), read transposed with
// ds_read_b64_tr_b16; LDS rows of 16-byte units XOR-swizzled (lds_tiles.hpp).
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "lookback.hpp"

namespace la {
namespace fused32 {

using namespace la::fused;

constexpr int NT = 256;          // threads per workgroup (4 wavefronts)
constexpr int CH = 64;           // chunk length
constexpr int TB = 256;          // tokens per block
constexpr int NCH = TB / CH;

template <int D, int M>
struct alignas(16) Smem {
  bf16_t Kh[CH * D];  // phi(K) of the current chunk, head and tail [CH][D]
  bf16_t Kl[CH * D];
  bf16_t Vh[CH * M];  // V of the current chunk, head and tail [CH][M]
  bf16_t Vl[CH * M];
  bf16_t Sh[M * D];   // R_c^T, head and tail [M][D]
  bf16_t Sl[M * D];
  bf16_t Zh[D];       // z of R_c, head and tail
  bf16_t Zl[D];
  int status;
};

// Eight floats -> bf16 head and tail units (round to nearest even).
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, u32x4& h, u32x4& l) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = cvt_pk(x[2 * i], x[2 * i + 1]);
    l[i] = cvt_pk(x[2 * i] - lo_of(h[i]), x[2 * i + 1] - hi_of(h[i]));
  }
}
__device__ __forceinline__ f32x4 phi4(const f32x4& x) { return f32x4{phi(x[0]), phi(x[1]), phi(x[2]), phi(x[3])}; }

// c + a b for head/tail operands.
__device__ __forceinline__ f32x4 mma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl, f32x4 c) {
  c = mma(ah, bh, c);
  c = mma(ah, bl, c);
  return mma(al, bh, c);
}

// A chunk's keys and values as raw registers: 8 consecutive floats per unit.
template <int D, int M>
struct RawKV {
  static constexpr int KU = CH * (D / 8) / NT, VU = CH * (M / 8) / NT;
  f32x4 k[KU][2], v[VU][2];
};

template <int D, int M, bool NTMP>
__device__ __forceinline__ void load_kv(RawKV<D, M>& r, const float* kh, const float* vh, int t0, int ntok, int tid) {
  using RR = RawKV<D, M>;
  constexpr int UK = D / 8, UV = M / 8;
  // Rows past the end of the sequence re-read its last row (no condition on the
  // load; they are zeroed when staged).
#pragma unroll
  for (int i = 0; i < RR::KU; ++i) {
    const int p = tid + NT * i, t = min(p / UK, ntok - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(kh + (size_t)(t0 + t) * D + (p % UK) * 8);
    r.k[i][0] = NTMP ? __builtin_nontemporal_load(src) : src[0];
    r.k[i][1] = NTMP ? __builtin_nontemporal_load(src + 1) : src[1];
  }
#pragma unroll
  for (int i = 0; i < RR::VU; ++i) {
    const int p = tid + NT * i, t = min(p / UV, ntok - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(vh + (size_t)(t0 + t) * M + (p % UV) * 8);
    r.v[i][0] = NTMP ? __builtin_nontemporal_load(src) : src[0];
    r.v[i][1] = NTMP ? __builtin_nontemporal_load(src + 1) : src[1];
  }
}

// phi(K) and V of a chunk (tokens t0 .. t0 + 63 of the head, ntok valid from t0)
// into the head/tail tiles; keys and values past the end become 0.
template <int D, int M>
__device__ __forceinline__ void stage_kv(Smem<D, M>& sm, const RawKV<D, M>& r, int nvalid, int tid, uint32_t l_kst,
                                         uint32_t l_vst) {
  using RR = RawKV<D, M>;
  constexpr int UK = D / 8, UV = M / 8;
  const f32x4 z4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RR::KU; ++i) {
    const bool ok = (tid + NT * i) / UK < nvalid;
    u32x4 hv, lv;
    split8(ok ? phi4(r.k[i][0]) : z4, ok ? phi4(r.k[i][1]) : z4, hv, lv);
    *reinterpret_cast<u32x4*>(tile_at<UK>(sm.Kh, l_kst, i * (NT / UK), 0)) = hv;
    *reinterpret_cast<u32x4*>(tile_at<UK>(sm.Kl, l_kst, i * (NT / UK), 0)) = lv;
  }
#pragma unroll
  for (int i = 0; i < RR::VU; ++i) {
    const bool ok = (tid + NT * i) / UV < nvalid;
    u32x4 hv, lv;
    split8(ok ? r.v[i][0] : z4, ok ? r.v[i][1] : z4, hv, lv);
    *reinterpret_cast<u32x4*>(tile_at<UV>(sm.Vh, l_vst, i * (NT / UV), 0)) = hv;
    *reinterpret_cast<u32x4*>(tile_at<UV>(sm.Vl, l_vst, i * (NT / UV), 0)) = lv;
  }
}

// acc += phi(K_c)^T V_c (and z += colsum phi(K_c)) for this wave's tiles.
template <int D, int M>
__device__ __forceinline__ void chunk_update(Tiles<D, M>& acc, const Smem<D, M>& sm, int w, uint32_t l_trk_w,
                                             uint32_t l_trv_w) {
  using GG = G<D, M>;
  const bf16x8 ones = ones8();
#pragma unroll
  for (int s = 0; s < CH / 32; ++s) {
    const bf16x8 ah = jfrag_at<GG::UK>(sm.Kh, l_trk_w, 32 * s, 0);
    const bf16x8 al = jfrag_at<GG::UK>(sm.Kl, l_trk_w, 32 * s, 0);
#pragma unroll
    for (int u = 0; u < GG::TMW; ++u) {
      const bf16x8 bvh = jfrag_at<GG::UV>(sm.Vh, l_trv_w, 32 * s, 16 * GG::WPT * u);
      const bf16x8 bvl = jfrag_at<GG::UV>(sm.Vl, l_trv_w, 32 * s, 16 * GG::WPT * u);
      acc.S[u] = mma3(ah, al, bvh, bvl, acc.S[u]);
    }
    if (w < GG::TD) {
      acc.Z = mma(ah, ones, acc.Z);
      acc.Z = mma(al, ones, acc.Z);
    }
  }
}

// A state (this wave's tiles of S, and z) as the S^T head/tail operand tiles
// [M][D] and the z head/tail vectors.
template <int D, int M>
__device__ __forceinline__ void put_state(Smem<D, M>& sm, const Tiles<D, M>& t, int w, int n, int g, uint32_t l_wr) {
  using GG = G<D, M>;
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) {
    int tdd, tm;
    tile_coords<D, M>(w, u, tdd, tm);
    const f32x4& x = t.S[u];
    const uint32_t h0 = cvt_pk(x[0], x[1]), h1 = cvt_pk(x[2], x[3]);
    *reinterpret_cast<u32x2*>(tile_at<GG::UK>(sm.Sh, l_wr, 16 * tm, 16 * tdd)) = u32x2{h0, h1};
    *reinterpret_cast<u32x2*>(tile_at<GG::UK>(sm.Sl, l_wr, 16 * tm, 16 * tdd)) =
        u32x2{cvt_pk(x[0] - lo_of(h0), x[1] - hi_of(h0)), cvt_pk(x[2] - lo_of(h1), x[3] - hi_of(h1))};
  }
  if (w < GG::TD && n == 0) {
    const uint32_t h0 = cvt_pk(t.Z[0], t.Z[1]), h1 = cvt_pk(t.Z[2], t.Z[3]);
    *reinterpret_cast<u32x2*>(&sm.Zh[16 * w + 4 * g]) = u32x2{h0, h1};
    *reinterpret_cast<u32x2*>(&sm.Zl[16 * w + 4 * g]) =
        u32x2{cvt_pk(t.Z[0] - lo_of(h0), t.Z[1] - hi_of(h0)), cvt_pk(t.Z[2] - lo_of(h1), t.Z[3] - hi_of(h1))};
  }
}

// num^T += S^T phi(Q)^T and den += z . phi(q) for this wave's 16 query columns,
// from the operands written by put_state.
template <int D, int M>
__device__ __forceinline__ void state_read(f32x4 (&numT)[M / 16], f32x4& den, const Smem<D, M>& sm,
                                           const bf16x8 (&qfh)[D / 32], const bf16x8 (&qfl)[D / 32], int g,
                                           uint32_t l_rd) {
  using GG = G<D, M>;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
#pragma unroll
    for (int tm = 0; tm < GG::TM; ++tm) {
      const bf16x8 sh = as_bf16x8(*reinterpret_cast<const u32x4*>(tile_at<GG::UK>(sm.Sh, l_rd, 16 * tm, 32 * s)));
      const bf16x8 sl = as_bf16x8(*reinterpret_cast<const u32x4*>(tile_at<GG::UK>(sm.Sl, l_rd, 16 * tm, 32 * s)));
      numT[tm] = mma3(sh, sl, qfh[s], qfl[s], numT[tm]);
    }
    const bf16x8 zh = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.Zh[32 * s + 8 * g]));
    const bf16x8 zl = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.Zl[32 * s + 8 * g]));
    den = mma3(zh, zl, qfh[s], qfl[s], den);
  }
}

// Within the chunk: num^T += V^T A^T and den += 1^T A^T with the masked scores
// A^T[j][i] = phi(k_j).phi(q_i), j <= i, for this wave's queries i = 16 w + n.
template <int D, int M>
__device__ __forceinline__ void intra_chunk(f32x4 (&numT)[M / 16], f32x4& den, const Smem<D, M>& sm,
                                            const bf16x8 (&qfh)[D / 32], const bf16x8 (&qfl)[D / 32], int w, int n,
                                            int g, uint32_t l_rd, uint32_t l_trv) {
  using GG = G<D, M>;
  const bf16x8 ones = ones8();
  f32x4 at[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    at[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t <= w) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const bf16x8 kah = as_bf16x8(*reinterpret_cast<const u32x4*>(tile_at<GG::UK>(sm.Kh, l_rd, 16 * t, 32 * s)));
        const bf16x8 kal = as_bf16x8(*reinterpret_cast<const u32x4*>(tile_at<GG::UK>(sm.Kl, l_rd, 16 * t, 32 * s)));
        at[t] = mma3(kah, kal, qfh[s], qfl[s], at[t]);
      }
      if (t == w) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > n) at[t][r] = 0.f;
      }
    }
  }
  // A score tile pair is the B operand of a 32-key slab (lane (n, g) holds
  // column i = n at the j-slots of group g).
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (2 * s <= w) {
      u32x4 ph, pl;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4& a = at[2 * s + h];
        ph[2 * h] = cvt_pk(a[0], a[1]);
        ph[2 * h + 1] = cvt_pk(a[2], a[3]);
        pl[2 * h] = cvt_pk(a[0] - lo_of(ph[2 * h]), a[1] - hi_of(ph[2 * h]));
        pl[2 * h + 1] = cvt_pk(a[2] - lo_of(ph[2 * h + 1]), a[3] - hi_of(ph[2 * h + 1]));
      }
      const bf16x8 pfh = as_bf16x8(ph), pfl = as_bf16x8(pl);
#pragma unroll
      for (int tm = 0; tm < GG::TM; ++tm) {
        const bf16x8 avh = jfrag_at<GG::UV>(sm.Vh, l_trv, 32 * s, 16 * tm);
        const bf16x8 avl = jfrag_at<GG::UV>(sm.Vl, l_trv, 32 * s, 16 * tm);
        numT[tm] = mma3(avh, avl, pfh, pfl, numT[tm]);
      }
      den = mma(ones, pfh, den);
      den = mma(ones, pfl, den);
    }
  }
}

template <int D, int M, bool LOCAL>
__global__ __launch_bounds__(NT, 2) void causal_fused32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ o,
    int N, int nblk, int BH, const float* S0, const float* z0, float* S_out, float* z_out,
    unsigned long long* flags, char* agg_ws, char* incl_ws, unsigned long long epoch, unsigned long long spin_ticks,
    int incl_period) {
  using GG = G<D, M>;
  constexpr int UK = GG::UK, UV = GG::UV;
  constexpr int QV = D / 32;  // d-slabs of a query row
  __shared__ Smem<D, M> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  // Block-major order, as in the bf16 kernel: a block's predecessors have
  // smaller workgroup indices (and, with BH a multiple of 8, run on its XCD).
  const int b = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int t0 = b * TB, ntok = min(N, t0 + TB) - t0;
  const int nch = (ntok + CH - 1) / CH;
  const float* kh = k + (size_t)bh * N * D;
  const float* vh = v + (size_t)bh * N * M;
  const float* qh = q + (size_t)bh * N * D;
  const int xcc = LOCAL ? xcc_id() : 0;
  const int td = w % GG::TD;
  const uint32_t l_kst = lane_off<UK>(tid / UK, 8 * (tid % UK));
  const uint32_t l_vst = lane_off<UV>(tid / UV, 8 * (tid % UV));
  const uint32_t l_trv = lane_off<UV>(4 * g + (n >> 2), 4 * (n & 3));
  const uint32_t l_trk_w = lane_off<UK>(4 * g + (n >> 2), 4 * (n & 3)) ^ xor_off<UK>(16 * td);
  const uint32_t l_trv_w = l_trv ^ xor_off<UV>(16 * (w / GG::TD));
  const uint32_t l_rd = lane_off<UK>(n, 8 * g);
  const uint32_t l_wr = lane_off<UK>(n, 4 * g);

  // Queries: this wave's rows 16 w + n of a chunk, d-slots 32 s + 8 g .. + 7.
  auto load_q = [&](f32x4 (&dst)[QV][2], int c) {
    const int i = min(c * CH + 16 * w + n, ntok - 1);
#pragma unroll
    for (int s = 0; s < QV; ++s) {
      const f32x4* src = reinterpret_cast<const f32x4*>(qh + (size_t)(t0 + i) * D + 32 * s + 8 * g);
      dst[s][0] = __builtin_nontemporal_load(src);
      dst[s][1] = __builtin_nontemporal_load(src + 1);
    }
  };
  auto split_q = [&](const f32x4 (&r)[QV][2], bf16x8 (&qh_)[QV], bf16x8 (&ql_)[QV]) {
#pragma unroll
    for (int s = 0; s < QV; ++s) {
      u32x4 hq, lq;
      split8(phi4(r[s][0]), phi4(r[s][1]), hq, lq);
      qh_[s] = as_bf16x8(hq);
      ql_[s] = as_bf16x8(lq);
    }
  };
  float* ob = o + ((size_t)bh * N + t0) * M;
  // o_i = num_i / den_i for query i = 16 w + n of chunk c: lane (n, g) holds the
  // four consecutive columns 16 tm + 4 g .. + 3 of every m-tile, one 16-byte
  // store each.
  auto store_out = [&](const f32x4 (&numT)[GG::TM], float den, int c) {
    const int i = c * CH + 16 * w + n;
    if (i < ntok) {
      const float inv = 1.f / den;
      float* dst = ob + (size_t)i * M + 4 * g;
#pragma unroll
      for (int tm = 0; tm < GG::TM; ++tm)
        *reinterpret_cast<float4*>(dst + 16 * tm) =
            float4{numT[tm][0] * inv, numT[tm][1] * inv, numT[tm][2] * inv, numT[tm][3] * inv};
    }
  };

  // ---------------- pass 1: the block increment ----------------
  // All of the block's keys and values are loaded at once (ordinary loads, so
  // that pass 2 finds the lines in the caches), and the chunks are taken in
  // the order 1, 2, .., then 0, so that chunk 0's tiles are still in LDS when
  // the pass ends.  Load slots past the last chunk re-read it (unused).
  auto chunk_at = [&](int i) { return i + 1 < nch ? i + 1 : 0; };
  Tiles<D, M> L;
  tiles_zero<D, M>(L);
  RawKV<D, M> r1[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = i < nch ? chunk_at(i) : nch - 1;
    load_kv<D, M, false>(r1[i], kh, vh, t0 + c * CH, ntok - c * CH, tid);
    __builtin_amdgcn_sched_barrier(0);  // keep the chunks' loads in order
  }
  f32x4 rq0[QV][2];
  if (o) load_q(rq0, 0);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (i >= nch) break;
    if (i > 0) __syncthreads();  // the previous chunk's tiles are read
    stage_kv<D, M>(sm, r1[i], ntok - chunk_at(i) * CH, tid, l_kst, l_vst);
    __syncthreads();
    chunk_update<D, M>(L, sm, w, l_trk_w, l_trv_w);
  }
  // Publish the increment; its stores drain while chunk 0's outputs within the
  // block are formed.  (Block 0 publishes its increment too when it publishes
  // no inclusive prefix.)
  const bool agg0 = b == 0 && incl_period > 1 && nblk > 1;
  if (b > 0 || agg0) agg_store<D, M, LOCAL, true>(agg_ws + ((size_t)bh * nblk + b) * GG::SLOT, L, w, lane, n, g);
  f32x4 numT0[GG::TM], den0{0.f, 0.f, 0.f, 0.f};
  bf16x8 qh0[QV], ql0[QV];
  if (o) {
    split_q(rq0, qh0, ql0);
#pragma unroll
    for (int tm = 0; tm < GG::TM; ++tm) numT0[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
    intra_chunk<D, M>(numT0, den0, sm, qh0, ql0, w, n, g, l_rd, l_trv);
  }

  // ---------------- phase 2: exclusive prefix of the block ----------------
  // Chunk 1 of pass 2 is loaded while the look-back waits.
  RawKV<D, M> r2[NCH];
  f32x4 rq[NCH][QV][2];
  Tiles<D, M> R;  // the running prefix of pass 2, from P
  block_prefix<D, M, LOCAL, true, 2>(R, L, sm.status, kh, vh, N, TB, b, bh, nblk, S0, z0, S_out, z_out, flags, agg_ws,
                                     incl_ws, epoch, spin_ticks, incl_period, agg0, xcc, tid, w, lane, n, g, [&] {
                                       if (o && nch > 1) {
                                         load_kv<D, M, true>(r2[1], kh, vh, t0 + CH, ntok - CH, tid);
                                         load_q(rq[1], 1);
                                         const int c2 = min(2, nch - 1);
                                         load_kv<D, M, true>(r2[2], kh, vh, t0 + c2 * CH, ntok - c2 * CH, tid);
                                         load_q(rq[2], c2);
                                       }
                                     });
  if (!o) return;

  // ---------------- pass 2: outputs, chunk by chunk ----------------
  const bool have_p = b > 0 || S0 != nullptr;
  // Chunk 0: its tiles are still in LDS; add the prefix of earlier blocks.
  if (have_p) {
    put_state<D, M>(sm, R, w, n, g, l_wr);  // nothing has read the state tiles yet
    __syncthreads();
    state_read<D, M>(numT0, den0, sm, qh0, ql0, g, l_rd);
  }
  store_out(numT0, den0[0], 0);
  if (nch > 1) chunk_update<D, M>(R, sm, w, l_trk_w, l_trv_w);  // R_1 = P + dS_0
#pragma unroll
  for (int c = 1; c < NCH; ++c) {
    if (c >= nch) break;
    __syncthreads();  // every wave has finished reading the previous chunk's tiles
    stage_kv<D, M>(sm, r2[c], ntok - c * CH, tid, l_kst, l_vst);
    put_state<D, M>(sm, R, w, n, g, l_wr);
    bf16x8 qfh[QV], qfl[QV];
    split_q(rq[c], qfh, qfl);
    if (c + 2 < NCH && c + 2 < nch) {
      load_kv<D, M, true>(r2[c + 2], kh, vh, t0 + (c + 2) * CH, ntok - (c + 2) * CH, tid);
      load_q(rq[c + 2], c + 2);
    }
    __syncthreads();
    f32x4 numT[GG::TM], den{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tm = 0; tm < GG::TM; ++tm) numT[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
    intra_chunk<D, M>(numT, den, sm, qfh, qfl, w, n, g, l_rd, l_trv);
    state_read<D, M>(numT, den, sm, qfh, qfl, g, l_rd);
    // R_{c+1} = R_c + dS_c (not needed after the last chunk).
    if (c + 1 < nch) chunk_update<D, M>(R, sm, w, l_trk_w, l_trv_w);
    store_out(numT, den[0], c);
  }
}

template <int D, int M>
static hipError_t fused32_impl(const void* q, const void* k, const void* v, void* o, int BH, int N, const float* S0,
                               const float* z0, float* S_out, float* z_out, void* ws, hipStream_t stream) {
  const int nblk = (N + TB - 1) / TB;
  const WsLayout l = layout<D, M>(BH, N, TB);
  char* base = (char*)ws;
  unsigned long long* flags = (unsigned long long*)base;
  char* agg = base + l.flags_bytes;
  char* incl = agg + (size_t)BH * nblk * l.slot_bytes;
  if (S0 && nblk > 1 && (S0 == S_out || z0 == z_out)) {
    // An in-place carry: block 0 reads the initial state while the last block
    // writes the final one; the kernel reads a private copy.
    float* S0c = (float*)(incl + (size_t)BH * nblk * l.slot_bytes);
    float* z0c = S0c + (size_t)BH * D * M;
    const long long nS = (long long)BH * D * M, nz = (long long)BH * D;
    const hipError_t e = launch_state_copy(S0, z0, S0c, z0c, nS, nz, stream);
    if (e != hipSuccess) return e;
    S0 = S0c;
    z0 = z0c;
  }
  // The look-back's wait bound, per launch: 200 us of the 100 MHz real-time
  // counter or LINATTN_LOOKBACK_SPIN_TICKS (0 sends every block whose
  // predecessors have not yet published to the fallback).
  const char* spin_env = getenv("LINATTN_LOOKBACK_SPIN_TICKS");
  const unsigned long long spin_ticks = spin_env ? strtoull(spin_env, nullptr, 10) : 20000ull;
  const dim3 grid((unsigned)nblk * (unsigned)BH), block(NT);
  // Inclusive prefixes on every second block of a head (every block when a
  // head has at most one block resident at a time).
#define LA_FUSED32_LAUNCH(LOC)                                                                                         \
  do {                                                                                                                 \
    const void* fn = (const void*)causal_fused32_kernel<D, M, LOC>;                                                    \
    const int period = std::min(2, std::max(1, resident_wgs(fn, NT) / std::max(BH, 1)));                              \
    hipLaunchKernelGGL((causal_fused32_kernel<D, M, LOC>), grid, block, 0, stream, (const float*)q, (const float*)k,   \
                       (const float*)v, (float*)o, N, nblk, BH, S0, z0, S_out, z_out, flags, agg, incl,                \
                       lookback_epoch(), spin_ticks, period);                                                          \
  } while (0)
  if (BH % 8 == 0) LA_FUSED32_LAUNCH(true);
  else LA_FUSED32_LAUNCH(false);
#undef LA_FUSED32_LAUNCH
  return hipGetLastError();
}

}  // namespace fused32

size_t causal_fused32_ws_bytes(int BH, int N, int D, int M) {
  using namespace fused32;
  if (BH <= 0 || N <= 0) return 0;
  switch (D * 100 + M) {
    case 3232: return layout<32, 32>(BH, N, TB).total;
    case 3264: return layout<32, 64>(BH, N, TB).total;
    case 6432: return layout<64, 32>(BH, N, TB).total;
    case 6464: return layout<64, 64>(BH, N, TB).total;
    default: return 0;
  }
}

hipError_t launch_causal_fused32(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                                 const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                                 hipStream_t stream) {
  using namespace fused32;
  switch (D * 100 + M) {
    case 3232: return fused32_impl<32, 32>(q, k, v, o, BH, N, S0, z0, S_out, z_out, ws, stream);
    case 3264: return fused32_impl<32, 64>(q, k, v, o, BH, N, S0, z0, S_out, z_out, ws, stream);
    case 6432: return fused32_impl<64, 32>(q, k, v, o, BH, N, S0, z0, S_out, z_out, ws, stream);
    case 6464: return fused32_impl<64, 64>(q, k, v, o, BH, N, S0, z0, S_out, z_out, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
